// Large-shape GEMM for per-row scales: 256 x 256 output tile per workgroup,
// four waves of 128 x 128, int32 accumulators in AGPRs (this translation
// unit is built without the VGPR accumulator form).
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part plus an
// 8-bit outlier part over reordered channels; Key points item 5: symmetric
// scales factor out of the integer sums) and the QUIK abstract (hybrid
// 4-bit layer with higher-precision outliers). With one scale per row and
// one per column for the INT4 head (and for the INT8 tail), the whole K loop
// accumulates exact integers and dequantization happens once per output.
//
// CDNA4 design (see gemm_kernels.hip for the widening and the LDS layout,
// which are shared)
// * A wave owns 4 x 4 blocks of 32 x 32, so each widened operand fragment
//   feeds four MFMAs: 3 VALU ops per v_mfma_i32_32x32x32_i8 for the nibble
//   widening, below what a lone wave can issue beside its MFMAs. The 256
//   accumulator registers are AGPRs, written by the MFMAs directly; one wave
//   per SIMD.
// * K-tiles of 64 bytes per row (128 INT4 channels) reach a 4-stage LDS ring
//   (32 KB per stage) by direct global->LDS DMA, prefetch distance 2, one
//   barrier per tile.
// * The INT8 outlier tail (at most four K-tiles) is loaded last and kept in
//   the ring whole; the epilogue multiplies it block by block into a 16-
//   register accumulator, so the tail needs no second 256-register set.
// * y = fp16(acc8 * (sa8 * sw8) + acc4 * (sa4 * sw4 / 256)), rows and columns
//   guarded at the ragged edges.
#include <algorithm>

#include "w4a4.h"
#include "gemm_common.h"

namespace w4a4 {
namespace gemm_big_impl {

using namespace gemm_impl;

constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128, FM = 4, FN = 4;
constexpr int STAGES = 4, PREFETCH = 2;
constexpr int A_BYTES = BM * kTileBytes, B_BYTES = BN * kTileBytes;
constexpr int STAGE = A_BYTES + B_BYTES;                 // 32 KB
constexpr int DA = BM * 4 / kThreads, DB = BN * 4 / kThreads;
constexpr int D = DA + DB;                               // DMA instructions per tile per lane
constexpr int MAX_TAIL_TILES = STAGES;

// One INT4 K-tile: two sub-steps of two 32-channel k-steps each.
__device__ __forceinline__ void mma_int4(v16i (&acc)[FM][FN], const unsigned char *st, int wm, int wn, int li,
                                         int lh) {
    const unsigned char *sA = st, *sB = st + A_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + lh;
        uint4 pa[FM], pb[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            pa[fm] = *reinterpret_cast<const uint4 *>(sA + swz(wm * WTM + fm * 32 + li, c));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            pb[fn] = *reinterpret_cast<const uint4 *>(sB + swz(wn * WTN + fn * 32 + li, c));
        v4i xa0[FM], xa1[FM], wb0[FN], wb1[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            xa0[fm] = v4i{(int)nib_lo(pa[fm].x), (int)nib_hi(pa[fm].x), (int)nib_lo(pa[fm].y), (int)nib_hi(pa[fm].y)};
            xa1[fm] = v4i{(int)nib_lo(pa[fm].z), (int)nib_hi(pa[fm].z), (int)nib_lo(pa[fm].w), (int)nib_hi(pa[fm].w)};
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            wb0[fn] = v4i{(int)nib_lo(pb[fn].x), (int)nib_hi(pb[fn].x), (int)nib_lo(pb[fn].y), (int)nib_hi(pb[fn].y)};
            wb1[fn] = v4i{(int)nib_lo(pb[fn].z), (int)nib_hi(pb[fn].z), (int)nib_lo(pb[fn].w), (int)nib_hi(pb[fn].w)};
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa0[fm], wb0[fn], acc[fm][fn], 0, 0, 0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa1[fm], wb1[fn], acc[fm][fn], 0, 0, 0);
    }
}

template <bool EXPORT>
__global__ __launch_bounds__(kThreads) void gemm_big_kernel(GemmArgs a) {
    __shared__ __align__(16) unsigned char lds[STAGES * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lh = lane >> 5;

    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    const int T4 = (int)(a.pitch4 / kTileBytes);   // INT4 K-tiles: ring tiles 0 .. T4-1
    const int T8 = (int)(a.pitch8 / kTileBytes);   // tail K-tiles: ring tiles T4 .. T-1
    const int T = T4 + T8;

    // ---- DMA sources of this lane (as in the 128 x 128 kernel) ------------------
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // INT4 offsets are kept; the tail's (used for at most four tiles) are
    // recomputed from the row when needed.
    uint32_t a4o[DA], b4o[DB];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int q = j * kThreads + tid;
        a4o[j] = min(row0 + (q >> 2), a.M - 1) * (uint32_t)a.pitch4 + dma_chunk_offset(q);
    }
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int q = j * kThreads + tid;
        b4o[j] = min(col0 + (q >> 2), a.N - 1) * (uint32_t)a.pitch4 + dma_chunk_offset(q);
    }
    auto issue = [&](int tt) {
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE;
        const uint32_t sa = st + wave_u * 1024, sb = st + A_BYTES + wave_u * 1024;
        if (tt < T4) {
            const uint8_t *A = a.a4 + tt * kTileBytes;
            const uint8_t *B = a.w4 + tt * kTileBytes;
#pragma unroll
            for (int j = 0; j < DA; ++j)
                dma16(A, a4o[j], sa + j * 4096);
#pragma unroll
            for (int j = 0; j < DB; ++j)
                dma16(B, b4o[j], sb + j * 4096);
        } else {
            const uint8_t *A = reinterpret_cast<const uint8_t *>(a.a8) + (tt - T4) * kTileBytes;
            const uint8_t *B = reinterpret_cast<const uint8_t *>(a.w8) + (tt - T4) * kTileBytes;
#pragma unroll
            for (int j = 0; j < DA; ++j) {
                const int q = j * kThreads + tid;
                dma16(A, min(row0 + (q >> 2), a.M - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q), sa + j * 4096);
            }
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                const int q = j * kThreads + tid;
                dma16(B, min(col0 + (q >> 2), a.N - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q), sb + j * 4096);
            }
        }
    };

    // ---- main loop over the INT4 tiles ------------------------------------------------
#pragma unroll
    for (int p = 0; p < PREFETCH; ++p)
        if (p < T)
            issue(p);
    v16i acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[fm][fn][r] = 0;
    for (int tt = 0; tt < T4; ++tt) {
        compiler_fence();
        if (tt + PREFETCH < T) {
            issue(tt + PREFETCH);
            __builtin_amdgcn_s_waitcnt(vmcnt_only(PREFETCH * D));
        } else {
            wait_tiles<D>(T - 1 - tt);
        }
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        mma_int4(acc, lds + (tt % STAGES) * STAGE, wm, wn, li, lh);
    }

    // ---- the whole tail into the ring --------------------------------------------------
    // Tiles [T4, min(T, T4 + PREFETCH)) are in flight already; the rest go to
    // ring slots whose last readers have all passed this barrier.
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    for (int tt = T4 + PREFETCH; tt < T; ++tt)
        issue(tt);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();

    // ---- epilogue, block by block ---------------------------------------------------------
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int mbase = row0 + wm * WTM + fm * 32 + lh * 4;   // row of element r: mbase + (r/4)*8 + r%4
        // this block row's tail operands, all tail tiles
        uint4 pa8[MAX_TAIL_TILES][2];
#pragma unroll
        for (int j = 0; j < MAX_TAIL_TILES; ++j)
            if (j < T8)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    pa8[j][s] = *reinterpret_cast<const uint4 *>(lds + ((T4 + j) % STAGES) * STAGE +
                                                                 swz(wm * WTM + fm * 32 + li, 2 * s + lh));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = col0 + wn * WTN + fn * 32 + li;
            v16i acc8 = zero;
#pragma unroll
            for (int j = 0; j < MAX_TAIL_TILES; ++j)
                if (j < T8)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const uint4 pb = *reinterpret_cast<const uint4 *>(
                            lds + ((T4 + j) % STAGES) * STAGE + A_BYTES + swz(wn * WTN + fn * 32 + li, 2 * s + lh));
                        const v4i x = {(int)pa8[j][s].x, (int)pa8[j][s].y, (int)pa8[j][s].z, (int)pa8[j][s].w};
                        const v4i w = {(int)pb.x, (int)pb.y, (int)pb.z, (int)pb.w};
                        acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x, w, acc8, 0, 0, 0);
                    }
            if constexpr (EXPORT) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = mbase + (r / 4) * 8 + (r % 4);
                    if (m < a.M && n < a.N) {
                        const int64_t e = (int64_t)m * a.N + n;
                        a.acc4_out[e] = acc[fm][fn][r] >> 8;
                        if (a.acc8_out)
                            a.acc8_out[e] = acc8[r];
                    }
                }
            } else {
                const int nc = min(n, a.N - 1);
                const float cs4 = a.sw4[(int64_t)nc * a.G] * (1.0f / 256.0f);
                const float cs8 = T8 > 0 ? a.sw8[nc] : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = mbase + (r / 4) * 8 + (r % 4);
                    const int mc = min(m, a.M - 1);
                    float y = 0.0f;
                    if (T8 > 0)
                        y += (float)acc8[r] * (a.sa8[mc] * cs8);
                    y += (float)acc[fm][fn][r] * (a.sa4[(int64_t)mc * a.G] * cs4);
                    if (m < a.M && n < a.N)
                        a.y[(int64_t)m * a.ldy + n] = (_Float16)y;
                }
            }
        }
    }
}

}  // namespace gemm_big_impl

using namespace gemm_big_impl;

bool gemm_big_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t G) {
    const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return G == 1 && K_n > 0 && w4a4_pitch8_bytes(n_out) / kTileBytes <= MAX_TAIL_TILES && tiles >= 256;
}

hipError_t launch_gemm_big(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (export_acc)
        hipLaunchKernelGGL(gemm_big_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_big_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
