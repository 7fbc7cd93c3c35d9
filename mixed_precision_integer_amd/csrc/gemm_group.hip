// GEMM for group-wise scales of 128 channels: 128 x 128 output tile per
// workgroup, four waves of 64 x 64, int32 accumulators in VGPRs, two
// workgroups per CU (two waves per SIMD).
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part with group
// quantization plus an 8-bit outlier part over reordered channels; Key points
// item 5: symmetric scales factor out of the integer sums, so each group's
// integer dot products are scaled once by the product of the row's and the
// column's group scale) and the QUIK abstract.
//
// CDNA4 design
// * With 128-channel groups every K-tile (64 bytes of each row = 128 INT4
//   channels) is one scale group: its 16 i8 MFMAs per wave start from a zero
//   C operand and the int32 sums are folded into fp32 accumulators,
//   y += float(acc) * (sa[m, t] * sw[n, t] / 256).
// * The per-element scale products come from the matrix core: one
//   v_mfma_f32_32x32x1_2b_f32 forms the outer products of two (row scales,
//   column scales) vector pairs as two 32 x 32 blocks, exact fp32 products in
//   the accumulator layout of the i8 MFMAs. Two of them cover a wave's four
//   blocks, so the dequantization costs a conversion and an FMA per element.
// * The weight fragment is the i8 MFMA's first operand: lane (li, lh) of
//   block (fm, fn) holds output row li and the columns 8 (r / 4) + 4 lh + r % 4,
//   so the fp16 result leaves as 8-byte stores of four consecutive columns.
// * Operands reach LDS by direct global->LDS DMA (same swizzled 64-byte rows
//   as the other GEMM kernels) into a 4-stage ring, three tiles ahead of the
//   MFMAs, with the tile's group scales (one float per row and per column)
//   riding along; ring tiles past the last one reload it, so every iteration
//   issues the same DMA and waits for the same count.
// * The INT8 outlier tail comes first, as one more group (per-row scales).
#include <algorithm>

#include "w4a4.h"
#include "gemm_common.h"

namespace w4a4 {
namespace gemm_group_impl {

using namespace gemm_impl;

typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int BM = 128, BN = 128, WT = 64, F = 2;    // tile, wave tile, 32 x 32 blocks per wave side
constexpr int STAGES = 4, PREFETCH = 3;                // ring tiles in flight ahead of the one in use
constexpr int A_BYTES = BM * kTileBytes, B_BYTES = BN * kTileBytes, S_BYTES = (BM + BN) * 4;
constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
constexpr int DA = BM * 4 / kThreads, DB = BN * 4 / kThreads;
constexpr int D = DA + DB + 1;                         // DMA instructions per tile per lane
static_assert(DA == 2 && DB == 2, "two 16-byte DMA rounds per operand");
static_assert(BM + BN == kThreads, "one scale per lane per tile");

// The four i8 MFMAs of one 32-channel k-step over the wave's 2 x 2 blocks.
__device__ __forceinline__ void mma_k(v16i (&acc)[F][F], const v4i (&x)[F], const v4i (&w)[F], bool fresh) {
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int fm = 0; fm < F; ++fm)
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[fn], x[fm], fresh ? zero : acc[fm][fn], 0, 0, 0);
}

// y += float(acc) * S for two of the wave's blocks: S holds the scale
// products of block (0, c) in registers 0-15 and of block (1, 1 - c) in 16-31.
template <int C>
__device__ __forceinline__ void fold_half(float (&y)[F][F][16], const v16i (&acc)[F][F], const v32f &S) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        y[0][C][r] = __builtin_fmaf((float)acc[0][C][r], S[r], y[0][C][r]);
        y[1][1 - C][r] = __builtin_fmaf((float)acc[1][1 - C][r], S[16 + r], y[1][1 - C][r]);
    }
}

// Accumulator export (test path): the exact integer sums of one group of a
// wave's 2 x 2 blocks; lane (li, lh) of block (fm, fn) holds token row li and
// the columns 8 (r / 4) + 4 lh + r % 4. This workgroup owns every sum of the
// group for its tile, so the adds never meet another workgroup's.
__device__ __forceinline__ void export_sums(const v16i (&acc)[F][F], int32_t *dst, int shift, const GemmArgs &a,
                                            int row0, int col0, int wm, int wn, int li, int lh) {
#pragma unroll
    for (int fm = 0; fm < F; ++fm) {
        const int m = row0 + wm * WT + fm * 32 + li;
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = col0 + wn * WT + fn * 32 + 8 * (r / 4) + 4 * lh + r % 4;
                if (m < a.M && n < a.N)
                    export_add(dst + (int64_t)m * a.N + n, acc[fm][fn][r] >> shift);
            }
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    compiler_fence();
}

template <bool EXPORT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_group_kernel(GemmArgs a) {
    __shared__ __align__(16) unsigned char lds[STAGES * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lh = lane >> 5;

    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    const int T8 = (int)(a.pitch8 / kTileBytes);    // tail tiles: ring tiles 0 .. T8-1
    const int T4 = (int)(a.pitch4 / kTileBytes);    // INT4 tiles (one group each): T8 .. T-1
    const int T = T8 + T4;

    // ---- DMA sources of this lane: slot q = j * 256 + tid of an operand holds
    // row q / 4, chunk (q % 4) ^ f(row) (the swizzle of the LDS reads)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t oa4[DA], oa8[DA], ob4[DB], ob8[DB];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int q = j * kThreads + tid;
        const uint32_t ra = min(row0 + (q >> 2), a.M - 1), rb = min(col0 + (q >> 2), a.N - 1);
        oa4[j] = ra * (uint32_t)a.pitch4 + dma_chunk_offset(q);
        oa8[j] = ra * (uint32_t)a.pitch8 + dma_chunk_offset(q);
        ob4[j] = rb * (uint32_t)a.pitch4 + dma_chunk_offset(q);
        ob8[j] = rb * (uint32_t)a.pitch8 + dma_chunk_offset(q);
    }
    // Scale slot of this lane: rows of the tile first (waves 0 and 1), then
    // its columns (waves 2 and 3), so the scale array is wave-uniform and the
    // per-lane byte offsets are fixed for the whole K loop.
    const bool wrow = wave_u < BM / 64;
    const int64_t sidx = wrow ? min(row0 + tid, a.M - 1) : min(col0 + tid - BM, a.N - 1);
    const uint32_t so4 = (uint32_t)(sidx * a.G) * 4u, so8 = (uint32_t)sidx * 4u;
    const float *s4base = wrow ? a.sa4 : a.sw4;
    const float *s8base = wrow ? a.sa8 : a.sw8;            // not read when T8 == 0

    // Ring tile tt: tail tile tt (tt < T8), INT4 tile tt - T8, or past the end
    // a reload of the last tile into a stage that is not read again. Every
    // DMA operand register is loop-invariant (see dma4s).
    auto issue = [&](int tt) {
        const int t = min(tt, T - 1);
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE;
        if (t < T8) {
            const uint8_t *A = reinterpret_cast<const uint8_t *>(a.a8) + t * kTileBytes;
            const uint8_t *B = reinterpret_cast<const uint8_t *>(a.w8) + t * kTileBytes;
#pragma unroll
            for (int j = 0; j < DA; ++j)
                dma16(A, oa8[j], st + j * 4096 + wave_u * 1024);
#pragma unroll
            for (int j = 0; j < DB; ++j)
                dma16(B, ob8[j], st + A_BYTES + j * 4096 + wave_u * 1024);
            dma4s(s8base, so8, st + A_BYTES + B_BYTES + wave_u * 256);
        } else {
            const uint8_t *A = a.a4 + (t - T8) * kTileBytes;
            const uint8_t *B = a.w4 + (t - T8) * kTileBytes;
#pragma unroll
            for (int j = 0; j < DA; ++j)
                dma16(A, oa4[j], st + j * 4096 + wave_u * 1024);
#pragma unroll
            for (int j = 0; j < DB; ++j)
                dma16(B, ob4[j], st + A_BYTES + j * 4096 + wave_u * 1024);
            dma4s(s4base + (t - T8), so4, st + A_BYTES + B_BYTES + wave_u * 256);
        }
    };

    float y[F][F][16];
#pragma unroll
    for (int fm = 0; fm < F; ++fm)
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                y[fm][fn][r] = 0.0f;
    v16i acc[F][F];

    // The same for ring tiles that are never tail tiles (the INT4 loop).
    auto issue4 = [&](int tt) {
        const int t4 = min(tt, T - 1) - T8;
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE;
        const uint8_t *A = a.a4 + t4 * kTileBytes;
        const uint8_t *B = a.w4 + t4 * kTileBytes;
#pragma unroll
        for (int j = 0; j < DA; ++j)
            dma16(A, oa4[j], st + j * 4096 + wave_u * 1024);
#pragma unroll
        for (int j = 0; j < DB; ++j)
            dma16(B, ob4[j], st + A_BYTES + j * 4096 + wave_u * 1024);
        dma4s(s4base + t4, so4, st + A_BYTES + B_BYTES + wave_u * 256);
    };

    // raw fragments of one ring tile (both sub-steps) and its three scales
    uint4 ra[2][F], rb[2][F];
    float rs, ca, cb;
    auto read_tile = [&](int tt) {
        const unsigned char *st = lds + (tt % STAGES) * STAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int f = 0; f < F; ++f) {
                ra[s][f] = *reinterpret_cast<const uint4 *>(st + swz(wm * WT + f * 32 + li, 2 * s + lh));
                rb[s][f] = *reinterpret_cast<const uint4 *>(st + A_BYTES + swz(wn * WT + f * 32 + li, 2 * s + lh));
            }
        const float *sS = reinterpret_cast<const float *>(st + A_BYTES + B_BYTES);
        rs = sS[wm * WT + lh * 32 + li];               // row scale of block fm = lh
        ca = sS[BM + wn * WT + lh * 32 + li];          // column scale of block fn = lh
        cb = sS[BM + wn * WT + (1 - lh) * 32 + li];    // column scale of block fn = 1 - lh
    };
    // wait for ring tile tt + 1 (two more may stay in flight), barrier (every
    // wave is done with tile tt: its stage takes ring tile tt + 4), next reads
    auto next_tile = [&](int tt, bool int4_only) {
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(vmcnt_only((PREFETCH - 1) * D));
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (int4_only)
            issue4(tt + STAGES);
        else
            issue(tt + STAGES);
        compiler_fence();
        read_tile(tt + 1);
    };
    // y += float(acc) * (rs * unit) x (ca | cb): the scale products on the
    // matrix core, blocks (0,0) | (1,1) from the column scales ca, then
    // (0,1) | (1,0) from cb (one 32-register product live at a time)
    auto fold_group = [&](float r_scale, float c_a, float c_b) {
        const v32f z = {};
        const v32f S1 = __builtin_amdgcn_mfma_f32_32x32x1f32(c_a, r_scale, z, 0, 0, 0);
        fold_half<0>(y, acc, S1);
        const v32f S2 = __builtin_amdgcn_mfma_f32_32x32x1f32(c_b, r_scale, z, 0, 0, 0);
        fold_half<1>(y, acc, S2);
    };

#pragma unroll
    for (int p = 0; p <= PREFETCH; ++p)
        issue(p);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(PREFETCH * D));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    read_tile(0);

    // ---- the INT8 tail: one group over T8 tiles (raw int8 operands) -------------------
    // (accumulators cleared once: a run-time "first tile" choice of the C
    // operand would keep a second set of accumulator registers live)
    if (T8 > 0) {
#pragma unroll
        for (int fm = 0; fm < F; ++fm)
#pragma unroll
            for (int fn = 0; fn < F; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[fm][fn][r] = 0;
    }
    for (int tt = 0; tt < T8; ++tt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i x[F], w[F];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                x[f] = v4i{(int)ra[s][f].x, (int)ra[s][f].y, (int)ra[s][f].z, (int)ra[s][f].w};
                w[f] = v4i{(int)rb[s][f].x, (int)rb[s][f].y, (int)rb[s][f].z, (int)rb[s][f].w};
            }
            mma_k(acc, x, w, false);
        }
        const float r0 = rs, a0 = ca, b0 = cb;
        next_tile(tt, false);
        if (tt == T8 - 1) {
            if constexpr (EXPORT)
                export_sums(acc, a.acc8_out, 0, a, row0, col0, wm, wn, li, lh);
            fold_group(r0, a0, b0);
        }
    }

    // ---- INT4 tiles, one 128-channel group each ------------------------------------
    // The MFMAs of tile t run from registers; then the next tile's barrier,
    // DMA and LDS reads are issued, and tile t's scale products and fold run
    // while those reads are in flight.
    for (int tt = T8; tt < T; ++tt) {
        // one sub-step at a time: widen (the second sub-step's widening waits
        // for the first one's MFMAs to have read their operands), then the
        // eight MFMAs
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i x[2][F], w[2][F];                         // [k half][block]
#pragma unroll
            for (int f = 0; f < F; ++f) {
                x[0][f] = v4i{(int)nib_lo(ra[s][f].x), (int)nib_hi(ra[s][f].x), (int)nib_lo(ra[s][f].y), (int)nib_hi(ra[s][f].y)};
                x[1][f] = v4i{(int)nib_lo(ra[s][f].z), (int)nib_hi(ra[s][f].z), (int)nib_lo(ra[s][f].w), (int)nib_hi(ra[s][f].w)};
                w[0][f] = v4i{(int)nib_lo(rb[s][f].x), (int)nib_hi(rb[s][f].x), (int)nib_lo(rb[s][f].y), (int)nib_hi(rb[s][f].y)};
                w[1][f] = v4i{(int)nib_lo(rb[s][f].z), (int)nib_hi(rb[s][f].z), (int)nib_lo(rb[s][f].w), (int)nib_hi(rb[s][f].w)};
            }
            mma_k(acc, x[0], w[0], s == 0);
            mma_k(acc, x[1], w[1], false);
        }
        const float r0 = rs * (1.0f / 256.0f), a0 = ca, b0 = cb;
        next_tile(tt, true);
        if constexpr (EXPORT)
            export_sums(acc, a.acc4_out + (int64_t)(tt - T8) * a.M * a.N, 8, a, row0, col0, wm, wn, li, lh);
        fold_group(r0, a0, b0);
    }
    // the reloads past the last tile land in LDS this workgroup still owns
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    // ---- epilogue: fp16, four consecutive columns per 8-byte store ---------------------
    // Lane indices are re-derived from an opaque copy of the thread id, so no
    // epilogue address is computed before the K loop and held through it.
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int ewm = (etid >> 6) >> 1, ewn = (etid >> 6) & 1, eli = etid & 31, elh = (etid & 63) >> 5;
    const bool vec = ((reinterpret_cast<uintptr_t>(a.y) | (uintptr_t)(a.ldy * 2)) & 7) == 0;
#pragma unroll
    for (int fm = 0; fm < F; ++fm) {
        const int m = row0 + ewm * WT + fm * 32 + eli;
        if (m >= a.M)
            continue;
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = col0 + ewn * WT + fn * 32 + q * 8 + elh * 4;
                const float *v = &y[fm][fn][q * 4];
                _Float16 *dst = a.y + (int64_t)m * a.ldy + n;
                if (vec && n + 3 < a.N) {
                    const _Float16 h0 = (_Float16)v[0], h1 = (_Float16)v[1], h2 = (_Float16)v[2], h3 = (_Float16)v[3];
                    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                    *reinterpret_cast<uint2 *>(dst) = uint2{lo, hi};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N)
                            dst[e] = (_Float16)v[e];
                }
            }
    }
}

}  // namespace gemm_group_impl

using namespace gemm_group_impl;

bool gemm_group_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group) {
    (void)N;
    (void)n_out;
    return group == 128 && K_n >= 128 && M > 64;
}

hipError_t launch_gemm_group(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (export_acc)
        hipLaunchKernelGGL(gemm_group_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_group_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
