// Mixed-precision GEMM for gfx950: INT4 x INT4 head + INT8 x INT8 outlier
// tail, exact int32 accumulation on the i8 matrix cores, fp32 scale epilogue.
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part plus an 8-bit
// outlier part over reordered channels, group quantization; Key points item
// 5: symmetric scales factor out of the integer sums; Interesting ideas I1:
// the outlier block is contiguous, so it is just more K-tiles of the same
// loop) and the QUIK abstract (hybrid 4-bit layer with higher-precision
// outliers).
//
// CDNA4 design notes
// * CDNA4 has no INT4 matrix instruction, so packed nibbles are widened
//   exactly to int8 in registers: for a packed dword p,
//     hi = p & 0xF0F0F0F0         -> four int8 lanes holding 16 * q_odd
//     lo = (p << 4) & 0xF0F0F0F0  -> four int8 lanes holding 16 * q_even
//   (the sign comes for free from the two's complement nibble). Both
//   operands carry the factor 16, so the int32 accumulator holds 256 * acc,
//   which is exact while K_n * 64 * 256 < 2^31; the epilogue folds 2^-8 into
//   the fp32 scale and the accumulator export shifts right by 8.
// * The nibble order inside an MFMA operand does not have to follow the
//   channel order: a dot product is invariant under any permutation of K
//   applied to both operands, and A and B are unpacked identically, so the
//   widened lo/hi dwords are fed to v_mfma_i32_32x32x32_i8 as they come.
// * A K-tile is 64 bytes of every row: 128 INT4 channels or 64 INT8 tail
//   channels. Tail tiles run first on a separate set of int32 accumulators
//   (different scales), then the INT4 tiles. At the end of each scale group
//   the int32 accumulators are converted and added into fp32 accumulators.
// * LDS rows are 80 bytes (64 + 16 padding): a lane reads 16 bytes of its
//   row per 64 K-values, and the 16-byte row skew keeps the eight lanes of a
//   ds_read_b128 phase on distinct bank groups.
// * Double-buffered LDS: tile t+1 is fetched into registers while tile t is
//   multiplied; one barrier per tile.
#include "w4a4_internal.h"

namespace w4a4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTileBytes = 64;   // bytes of each row per K-tile
constexpr int kLdsPitch = 80;    // LDS bytes per row (64 data + 16 skew)

__device__ __forceinline__ uint32_t nib_hi(uint32_t p) { return p & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_lo(uint32_t p) { return (p << 4) & 0xF0F0F0F0u; }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool EXPORT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    constexpr int CA = BM * 4 / kThreads;       // 16-byte chunks per lane, A tile
    constexpr int CB = BN * 4 / kThreads;
    static_assert(CA >= 1 && CB >= 1 && BM <= kThreads && BN <= kThreads, "loader");
    constexpr int A_BYTES = BM * kLdsPitch, B_BYTES = BN * kLdsPitch;
    constexpr int STAGE = A_BYTES + B_BYTES + (BM + BN) * 4;

    __shared__ __align__(16) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;

    const int tiles_n = (a.N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int row0 = tm * BM, col0 = tn * BN;

    const int T8 = (int)(a.pitch8 / kTileBytes);
    const int T4 = (int)(a.pitch4 / kTileBytes);
    const int T = T8 + T4;
    const int tiles_per_group = a.group > 0 ? a.group / 128 : T4;

    // ---- tile loader state -------------------------------------------------
    uint4 ra[CA], rb[CB];
    float rsa = 0.0f, rsb = 0.0f;

    auto group_end = [&](int tt, int &gidx) -> bool {
        if (tt < T8) {
            gidx = -1;
            return tt == T8 - 1;
        }
        const int t4 = tt - T8;
        gidx = (t4 + 1) / tiles_per_group - 1;
        return (t4 + 1) % tiles_per_group == 0;
    };

    auto load_tile = [&](int tt) {
        const bool tail = tt < T8;
        const uint8_t *abase = tail ? reinterpret_cast<const uint8_t *>(a.a8) : a.a4;
        const uint8_t *bbase = tail ? reinterpret_cast<const uint8_t *>(a.w8) : a.w4;
        const int64_t pitch = tail ? a.pitch8 : a.pitch4;
        const int64_t koff = (int64_t)(tail ? tt : tt - T8) * kTileBytes;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * kThreads;
            const int r = min(row0 + c / 4, a.M - 1);
            ra[i] = *reinterpret_cast<const uint4 *>(abase + (int64_t)r * pitch + koff + (c % 4) * 16);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * kThreads;
            const int r = min(col0 + c / 4, a.N - 1);
            rb[i] = *reinterpret_cast<const uint4 *>(bbase + (int64_t)r * pitch + koff + (c % 4) * 16);
        }
        int gidx;
        if (!EXPORT && group_end(tt, gidx)) {
            const float *sa = tail ? a.sa8 : a.sa4;
            const float *sb = tail ? a.sw8 : a.sw4;
            const int stride = tail ? 1 : a.G;
            const int g = tail ? 0 : gidx;
            if (tid < BM)
                rsa = sa[(int64_t)min(row0 + tid, a.M - 1) * stride + g];
            if (tid < BN)
                rsb = sb[(int64_t)min(col0 + tid, a.N - 1) * stride + g];
        }
    };

    auto store_tile = [&](int tt, int stage) {
        unsigned char *sA = lds + stage * STAGE;
        unsigned char *sB = sA + A_BYTES;
        float *sS = reinterpret_cast<float *>(sB + B_BYTES);
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<uint4 *>(sA + (c / 4) * kLdsPitch + (c % 4) * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<uint4 *>(sB + (c / 4) * kLdsPitch + (c % 4) * 16) = rb[i];
        }
        int gidx;
        if (!EXPORT && group_end(tt, gidx)) {
            if (tid < BM)
                sS[tid] = rsa;
            if (tid < BN)
                sS[BM + tid] = rsb;
        }
    };

    // ---- accumulators ------------------------------------------------------
    v16i acc[FM][FN];
    float yacc[EXPORT ? 1 : FM][EXPORT ? 1 : FN][16];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            acc[fm][fn] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            if constexpr (!EXPORT) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    yacc[fm][fn][r] = 0.0f;
            }
        }

    // ---- main loop -----------------------------------------------------------
    if (T > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();

    for (int tt = 0; tt < T; ++tt) {
        const int stage = tt & 1;
        if (tt + 1 < T)
            load_tile(tt + 1);

        const unsigned char *sA = lds + stage * STAGE + (wm * WTM + li) * kLdsPitch + lh * 16;
        const unsigned char *sB = lds + stage * STAGE + A_BYTES + (wn * WTN + li) * kLdsPitch + lh * 16;
        const bool tail = tt < T8;

#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint4 pa[FM], pb[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                pa[fm] = *reinterpret_cast<const uint4 *>(sA + fm * 32 * kLdsPitch + s * 32);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                pb[fn] = *reinterpret_cast<const uint4 *>(sB + fn * 32 * kLdsPitch + s * 32);
            if (tail) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const v4i x = {(int)pa[fm].x, (int)pa[fm].y, (int)pa[fm].z, (int)pa[fm].w};
                        const v4i w = {(int)pb[fn].x, (int)pb[fn].y, (int)pb[fn].z, (int)pb[fn].w};
                        acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x, w, acc[fm][fn], 0, 0, 0);
                    }
            } else {
                v4i xa0[FM], xa1[FM], wb0[FN], wb1[FN];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    xa0[fm] = v4i{(int)nib_lo(pa[fm].x), (int)nib_hi(pa[fm].x),
                                  (int)nib_lo(pa[fm].y), (int)nib_hi(pa[fm].y)};
                    xa1[fm] = v4i{(int)nib_lo(pa[fm].z), (int)nib_hi(pa[fm].z),
                                  (int)nib_lo(pa[fm].w), (int)nib_hi(pa[fm].w)};
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    wb0[fn] = v4i{(int)nib_lo(pb[fn].x), (int)nib_hi(pb[fn].x),
                                  (int)nib_lo(pb[fn].y), (int)nib_hi(pb[fn].y)};
                    wb1[fn] = v4i{(int)nib_lo(pb[fn].z), (int)nib_hi(pb[fn].z),
                                  (int)nib_lo(pb[fn].w), (int)nib_hi(pb[fn].w)};
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa0[fm], wb0[fn], acc[fm][fn], 0, 0, 0);
                        acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa1[fm], wb1[fn], acc[fm][fn], 0, 0, 0);
                    }
            }
        }

        int gidx;
        if (group_end(tt, gidx)) {
            if constexpr (EXPORT) {
                int32_t *dst = tail ? a.acc8_out : a.acc4_out + (int64_t)gidx * a.M * a.N;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const int n = col0 + wn * WTN + fn * 32 + li;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = row0 + wm * WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                            const int v = acc[fm][fn][r];
                            if (m < a.M && n < a.N)
                                dst[(int64_t)m * a.N + n] = tail ? v : (v >> 8);
                            acc[fm][fn][r] = 0;
                        }
                    }
            } else {
                const float *sS = reinterpret_cast<const float *>(lds + stage * STAGE + A_BYTES + B_BYTES);
                const float unit = tail ? 1.0f : (1.0f / 256.0f);
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
                    for (int fn = 0; fn < FN; ++fn) {
                        const float cs = sS[BM + wn * WTN + fn * 32 + li] * unit;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            yacc[fm][fn][r] += (float)acc[fm][fn][r] * (rs[r] * cs);
                            acc[fm][fn][r] = 0;
                        }
                    }
                }
            }
        }

        if (tt + 1 < T)
            store_tile(tt + 1, stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: fp16 store -----------------------------------------------
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

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (export_acc)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true>), dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false>), dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    if (a.M == 0 || a.N == 0)
        return hipSuccess;
    if (a.M > 64)
        return launch_cfg<128, 128, 2, 2>(a, export_acc, stream);
    return launch_cfg<64, 128, 2, 2>(a, export_acc, stream);
}

}  // namespace w4a4
