// W4A8 GEMM for gfx950: INT8 activations (one scale per token) x INT4
// weights (one scale per output channel, or per group of a multiple of 128
// channels), exact int32 accumulation on the i8 matrix cores, fp32 scale
// epilogue, fp16 output.
//
// Method: the QQQ abstract on the "smoothquant" tag page (4-bit weights
// with 8-bit activations; a per-channel and a per-group W4A8 GEMM). The
// operands come from this
// library's own quantizer: activations are the INT8 rows it writes when every
// channel is an "outlier" in the identity order, weights the INT4 rows it
// writes with no outliers.
//
// CDNA4 design (shares the DMA, swizzle and tile-walk helpers of the W4A4
// GEMMs)
// * A K-tile is 128 channels: 128 bytes of every activation row (two 64-byte
//   sub-tiles, channels 0-63 and 64-127, each stored with the XOR-swizzled
//   16-byte chunk layout) and 64 bytes of every weight row.
// * The weight nibbles are widened exactly as in the W4A4 kernels (high
//   nibble in place, low nibble shifted up: int8 lanes holding 16 q), so a
//   16-byte weight chunk of 32 channels becomes two MFMA operands whose
//   lanes hold the channels in the order 0,2,4,6 | 1,3,5,7 | 8,10,.. | 9,11,..
//   The matching 32 activation bytes (two 16-byte chunks) are put in the
//   same order by one v_perm_b32 per output dword, so both operands of
//   v_mfma_i32_32x32x32_i8 pair the same channels. The accumulator holds
//   16 x the exact sum (|16 q_w q_a| <= 16384: exact while K * 16384 < 2^31);
//   the epilogue folds 1/16 into the fp32 scale and the export shifts by 4.
// * A three-stage LDS ring (prefetch distance 1) of 25 KB stages keeps two
//   workgroups on a CU; one barrier per tile, every wave waiting for its own
//   DMA with an explicit vmcnt first.
// * The group's scales ride along with every tile (one DMA dword per lane):
//   the token scales, then the weight scales of the tile's group.
#include <algorithm>

#include "gemm_common.h"
#include "w4a8_internal.h"

namespace w4a4 {
namespace w4a8_impl {

using gemm_impl::compiler_fence;
using gemm_impl::dma_chunk_offset;
using gemm_impl::kThreads;
using gemm_impl::nib_hi;
using gemm_impl::nib_lo;
using gemm_impl::swz;
using gemm_impl::v16i;
using gemm_impl::v4i;
using gemm_impl::vmcnt_only;

constexpr int BM = 128, BN = 128, WAVES_N = 2;
constexpr int WTM = 64, WTN = 64, FM = 2, FN = 2;
constexpr int STAGES = 3, PREFETCH = 1;
constexpr int SUB_BYTES = BM * 64;                 // one 64-channel activation sub-tile
constexpr int A_BYTES = 2 * SUB_BYTES, B_BYTES = BN * 64;
constexpr int S_BYTES = kThreads * 4;              // BM token scales + BN weight scales
constexpr int DA = 2 * BM * 4 / kThreads, DB = BN * 4 / kThreads, DS = 1;
static_assert(BM + BN == kThreads, "one scale per lane");

// bytes {0, 2} of lo and hi (even channels), or {1, 3} (odd channels)
__device__ __forceinline__ uint32_t even_bytes(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_perm(hi, lo, 0x06040200u);
}
__device__ __forceinline__ uint32_t odd_bytes(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_perm(hi, lo, 0x07050301u);
}

// The MFMAs of one K-tile in LDS stage `st`. FRESH: the tile opens a scale
// group (its first MFMAs take C = 0).
template <bool FRESH>
__device__ __forceinline__ void mma_tile(v16i (&acc)[FM][FN], const unsigned char *st, int wm, int wn, int li,
                                         int lh) {
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const unsigned char *sB = st + A_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + lh;                  // weight chunk: channels 32c .. 32c + 31
        const unsigned char *sA = st + (c >> 1) * SUB_BYTES;
        const int ca = (2 * c) & 3;                // activation chunks ca, ca + 1 of that sub-tile
        uint4 pb[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            pb[fn] = *reinterpret_cast<const uint4 *>(sB + swz(wn * WTN + fn * 32 + li, c));
        v4i xa0[FM], xa1[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * WTM + fm * 32 + li;
            const uint4 p0 = *reinterpret_cast<const uint4 *>(sA + swz(r, ca));
            const uint4 p1 = *reinterpret_cast<const uint4 *>(sA + swz(r, ca + 1));
            xa0[fm] = v4i{(int)even_bytes(p0.y, p0.x), (int)odd_bytes(p0.y, p0.x), (int)even_bytes(p0.w, p0.z),
                          (int)odd_bytes(p0.w, p0.z)};
            xa1[fm] = v4i{(int)even_bytes(p1.y, p1.x), (int)odd_bytes(p1.y, p1.x), (int)even_bytes(p1.w, p1.z),
                          (int)odd_bytes(p1.w, p1.z)};
        }
        const bool z = FRESH && s == 0;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const v4i wb0 = {(int)nib_lo(pb[fn].x), (int)nib_hi(pb[fn].x), (int)nib_lo(pb[fn].y),
                             (int)nib_hi(pb[fn].y)};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa0[fm], wb0, z ? zero : acc[fm][fn], 0, 0, 0);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const v4i wb1 = {(int)nib_lo(pb[fn].z), (int)nib_hi(pb[fn].z), (int)nib_lo(pb[fn].w),
                             (int)nib_hi(pb[fn].w)};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa1[fm], wb1, acc[fm][fn], 0, 0, 0);
        }
    }
}

// End of a scale group: y += float(acc) * (sa[m] * sw[n] / 16), the scales
// read from the LDS stage of the group's last tile.
__device__ __forceinline__ void dequant_group(const v16i (&acc)[FM][FN], float (&yacc)[FM][FN][16],
                                              const unsigned char *st, int wm, int wn, int li, int lh) {
    const float *sS = reinterpret_cast<const float *>(st + A_BYTES + B_BYTES);
    float cs[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        cs[fn] = sS[BM + wn * WTN + fn * 32 + li] * (1.0f / 16.0f);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        float rs[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(sS + wm * WTM + fm * 32 + q * 8 + lh * 4);
            rs[q * 4 + 0] = v.x;
            rs[q * 4 + 1] = v.y;
            rs[q * 4 + 2] = v.z;
            rs[q * 4 + 3] = v.w;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                yacc[fm][fn][r] += (float)acc[fm][fn][r] * (rs[r] * cs[fn]);
    }
}

__device__ __forceinline__ void export_group(const v16i (&acc)[FM][FN], const GemmArgs &a, int g, int row0,
                                             int col0, int wm, int wn, int li, int lh) {
    int32_t *dst = a.acc4_out + (int64_t)g * a.M * a.N;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = col0 + wn * WTN + fn * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = row0 + wm * WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                if (m < a.M && n < a.N)
                    dst[(int64_t)m * a.N + n] = acc[fm][fn][r] >> 4;
            }
        }
}

template <bool EXPORT>
__global__ __launch_bounds__(kThreads) void gemm_w4a8_kernel(GemmArgs a) {
    constexpr int STAGE = A_BYTES + B_BYTES + (EXPORT ? 0 : S_BYTES);
    constexpr int D = DA + DB + (EXPORT ? 0 : DS);   // DMA instructions per tile per lane
    __shared__ __align__(16) unsigned char lds[STAGES * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    gemm_impl::tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    const int T = (int)(a.pitch4 / 64);              // K-tiles of 128 channels
    const int tiles_per_group = a.group > 0 ? a.group / 128 : T;

    // per-lane DMA offsets, fixed for the whole K loop
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t ao[DA], bo[DB];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int h = j / (DA / 2);                  // activation sub-tile
        const int q = (j % (DA / 2)) * kThreads + tid, r = q >> 2;
        const uint32_t row = min(row0 + r, a.M - 1);
        ao[j] = row * (uint32_t)a.pitch8 + h * 64 + dma_chunk_offset(q);
    }
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int q = j * kThreads + tid, r = q >> 2;
        const uint32_t row = min(col0 + r, a.N - 1);
        bo[j] = row * (uint32_t)a.pitch4 + dma_chunk_offset(q);
    }
    const bool s_is_a = tid < BM;
    const uint32_t s_row = s_is_a ? min(row0 + tid, a.M - 1) : min(col0 + tid - BM, a.N - 1);

    auto issue = [&](int tt) {
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE;
        const uint8_t *A = reinterpret_cast<const uint8_t *>(a.a8) + tt * 128;
        const uint8_t *B = a.w4 + tt * 64;
#pragma unroll
        for (int j = 0; j < DA; ++j)
            dma16(A, ao[j], st + (j / (DA / 2)) * SUB_BYTES + (j % (DA / 2)) * 4096 + wave_u * 1024);
#pragma unroll
        for (int j = 0; j < DB; ++j)
            dma16(B, bo[j], st + A_BYTES + j * 4096 + wave_u * 1024);
        if constexpr (!EXPORT) {
            const int g = tt / tiles_per_group;
            dma4(s_is_a ? a.sa8 + s_row : a.sw4 + s_row * (uint32_t)a.G + g,
                 st + A_BYTES + B_BYTES + wave_u * 256);
        }
    };

    auto begin_tile = [&](int tt) -> const unsigned char * {
        compiler_fence();
        if (tt + PREFETCH < T) {
            issue(tt + PREFETCH);
            if constexpr (EXPORT)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // accumulator stores share vmcnt
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(PREFETCH * D));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        }
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        return lds + (tt % STAGES) * STAGE;
    };

    v16i acc[FM][FN];
    float yacc[FM][FN][16];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                yacc[fm][fn][r] = 0.0f;

#pragma unroll
    for (int p = 0; p < PREFETCH; ++p)
        if (p < T)
            issue(p);
    int tt = 0;
    while (tt < T) {
        const int g = tt / tiles_per_group;
        const int run_end = min((g + 1) * tiles_per_group, T);
        const unsigned char *st = begin_tile(tt++);
        mma_tile<true>(acc, st, wm, wn, li, lh);
        while (tt < run_end) {
            st = begin_tile(tt++);
            mma_tile<false>(acc, st, wm, wn, li, lh);
        }
        if constexpr (EXPORT)
            export_group(acc, a, g, row0, col0, wm, wn, li, lh);
        else
            dequant_group(acc, yacc, st, wm, wn, li, lh);
    }
    if constexpr (!EXPORT) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = col0 + wn * WTN + fn * 32 + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row0 + wm * WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                    if (m < a.M && n < a.N)
                        a.y[(int64_t)m * a.ldy + n] = (_Float16)yacc[fm][fn][r];
                }
            }
    }
}

}  // namespace w4a8_impl

hipError_t launch_gemm_w4a8(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    using namespace w4a8_impl;
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (export_acc)
        hipLaunchKernelGGL(gemm_w4a8_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_w4a8_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
