// FP6 decode GEMM: batches of 33..128 token rows with group scales of 128
// channels (the Llama-65B decode sweep's larger batches).
//
// Method: the layer of the QUIK abstract and the Atom summary page (Summary
// paragraph 2: INT4 groups of 128 channels with their own scales, 8-bit
// outliers; Key points item 5: symmetric scales factor out of the integer
// sums), here on gfx950's FP6 matrix instruction: E2M3 codes of q / 8 with a
// block scale of 8 on each operand give exact integer sums in fp32.
//
// Design (a decode batch reads each weight once from HBM; the tokens are
// small and shared by every workgroup, so they are served by L2):
// * A workgroup computes 32 output columns for all M <= 32 MB token rows.
//   Its eight waves take pairs of 32-row blocks times contiguous ranges of
//   the 128-channel groups, each adding its own partial y; the partials meet
//   in LDS in range order at the end (deterministic).
// * No LDS ring and no barrier in the main loop: the u6 layout puts one
//   operand fragment (a lane's row, 32 channels) at 16 + 8 contiguous bytes
//   of a 32-row block, so fragments are loaded straight into registers.
//   Tokens are requested three groups ahead and weights four (the token
//   requests go out first in each step, so waiting for a group's tokens never
//   waits for the weights requested after them).
// * Per group and row block: two FP6 MFMAs (the sum starts from zero), one
//   v_mfma_f32_32x32x2f32 forming the products sw[n] sa[m] in the
//   accumulator layout, and one FMA per element: y += sum * (sw sa).
// * The INT8 tail of row block b (at most four 64-channel tiles) runs on the
//   i8 matrix core in wave b, folded into that wave's partial y.
// * Export (test path): the exact sums of every group and of the tail, from
//   this main loop (each group belongs to one wave, so plain stores).
#include <algorithm>

#include "w4a4.h"
#include "gemm_fp6_common.h"
#include "gemm_fp6_internal.h"

namespace w4a4 {
namespace gemm_fp6_impl {

constexpr int kDWaves = 8, kDThreads = kDWaves * 64;
constexpr int kDBN = 32;                            // output columns per workgroup
constexpr int kDMaxGroups = 16;                     // groups per wave up to 128 rows (K_n <= 8192)

// One operand fragment of k-step t of a 32-row block: the lane's row li and
// 32-channel chunk lh (bytes 0..15 at 512 lh + 16 li, 16..23 at
// 1024 + 256 lh + 8 li).
__device__ __forceinline__ v6i fragment(const uint8_t *block_row, int t, uint32_t flo, uint32_t fhi) {
    const uint8_t *blk = block_row + (int64_t)t * BLK;
    return load_operand(blk + flo, blk + fhi);
}

// sum = w^T x (+ c): the eight-register operands of the builtin, of which FP6
// reads the first six
__device__ __forceinline__ v16f mma_fp6(const v6i &w, const v6i &x, const v16f &c) {
    typedef int v8i_t __attribute__((ext_vector_type(8)));
    v8i_t w8, x8;
    w8.s012345 = w;
    x8.s012345 = x;
    w8.s67 = v2i{0, 0};
    x8.s67 = v2i{0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, x8, c, 2, 2, 0, 130, 0, 130);
}

// Waves: RG pairs of row blocks times KS contiguous ranges of groups
// (RG * KS = 8). Wave w takes blocks 2 (w % RG) and 2 (w % RG) + 1 over
// range w / RG.
template <int MB, bool EXPORT>
__global__ __launch_bounds__(kDThreads) void gemm_fp6_decode_kernel(Fp6GemmArgs a) {
    constexpr int RG = (MB + 1) / 2, KS = kDWaves / RG;
    constexpr int GMAX = MB > 4 ? 2 * kDMaxGroups : kDMaxGroups;   // groups per wave (K_n <= 8192)
    static_assert(RG * KS == kDWaves, "waves split into block pairs and group ranges");
    // LDS: the scale tables during the main loop, then (after a barrier) the
    // partial blocks: red [block][range][register][lane]; sc per wave: sa of
    // its two blocks and sw, [32 rows][groups], rows padded by one
    constexpr int RED = MB * KS * 16 * 64, SC = kDWaves * 3 * 32 * (GMAX + 1);
    __shared__ float lds_f[RED > SC ? RED : SC];
    float *red = lds_f;
    float(*sc)[3][32][GMAX + 1] = reinterpret_cast<float(*)[3][32][GMAX + 1]>(lds_f);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int n0 = blockIdx.x * kDBN;
    const int rg = wave % RG, ks = wave / RG;
    const int b0 = 2 * rg;
    const int nb = min(2, MB - b0);                  // blocks of this wave (uniform)

    const int T = (int)(a.pitch4 / 32);             // k-steps of 64 channels
    const int G = T / 2;                            // groups of 128 channels
    const int T8 = (int)(a.pitch8 / kTileBytes);    // tail tiles of 64 channels
    const int gper = (G + KS - 1) / KS;             // <= GMAX (checked at launch)
    const int g0 = min(ks * gper, G);
    const int ng = min(g0 + gper, G) - g0;

    const uint32_t flo = 512u * lh + 16u * li, fhi = 1024u + 256u * lh + 8u * li;
    const uint8_t *Wb = a.w_u6 + (int64_t)(n0 / 32) * T * BLK;
    const uint8_t *Ab[2] = {a.a_u6 + (int64_t)b0 * T * BLK, a.a_u6 + (int64_t)min(b0 + 1, MB - 1) * T * BLK};
    const int64_t nrow = min(n0 + li, a.N - 1);
    const int64_t mrow[2] = {min(32 * b0 + li, a.M - 1), min(32 * (b0 + 1) + li, a.M - 1)};

    // The scales of the wave's rows and groups go to LDS first, in loads of
    // 16 consecutive groups of 4 rows (a scale per group and row would touch
    // 32 cache lines per load), for every group of the range
    float(*ws)[32][GMAX + 1] = sc[wave];
#pragma unroll
    for (int gc = 0; gc < GMAX / 16; ++gc) {       // 16 groups at a time
        const int gg = 16 * gc + (lane & 15);
        const int g = min(g0 + min(gg, max(ng - 1, 0)), G - 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (j < nb)
                    ws[j][r][gg] = a.sa4[min(32 * (b0 + j) + r, a.M - 1) * (int64_t)G + g];
            ws[2][r][gg] = a.sw4[min(n0 + r, a.N - 1) * (int64_t)G + g];
        }
    }

    // Group k of the range (clamped to the last one: the requests are issued
    // unconditionally, so the wait counts stay exact across the unrolled
    // steps; a clamped repeat is never used).
    v6i wf[GMAX][2], af[GMAX][2][2];
    auto load_w = [&](int k) {
        const int g = g0 + min(k, ng - 1), t = 2 * g;
        wf[k][0] = fragment(Wb, t, flo, fhi);
        wf[k][1] = fragment(Wb, t + 1, flo, fhi);
    };
    auto load_a = [&](int k) {
        const int g = g0 + min(k, ng - 1), t = 2 * g;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (j < nb) {
                af[k][j][0] = fragment(Ab[j], t, flo, fhi);
                af[k][j][1] = fragment(Ab[j], t + 1, flo, fhi);
            }
    };

    v16f y[2];
    y[0] = y[1] = v16f{};
    const v16f zf = {};

    // requests run PA groups ahead for the tokens and PW for the weights; in
    // every step the token requests go out first
    constexpr int PA = 2, PW = 3;
    if (ng > 0) {
#pragma unroll
        for (int k = 0; k < PA; ++k)
            load_a(k);
#pragma unroll
        for (int k = 0; k < PW; ++k)
            load_w(k);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < GMAX; ++k) {
            if (k + PA < GMAX)
                load_a(k + PA);
            if (k + PW < GMAX)
                load_w(k + PW);
            asm volatile("" ::: "memory");         // the requests go out here, not next to their use
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (j < nb) {
                    v16f acc = mma_fp6(wf[k][0], af[k][j][0], zf);
                    acc = mma_fp6(wf[k][1], af[k][j][1], acc);
                    if constexpr (EXPORT) {
                        const int m = 32 * (b0 + j) + li;
                        if (m < a.M) {
                            int32_t *dst = a.acc4_out + ((int64_t)(g0 + k) * a.M + m) * a.N + n0 + 4 * lh;
                            const int nl = a.N - n0 - 4 * lh;   // columns left from dst
#pragma unroll
                            for (int e = 0; e < 16; ++e)
                                if (8 * (e / 4) + e % 4 < nl)
                                    dst[8 * (e / 4) + e % 4] = (int32_t)acc[e];
                        }
                        asm volatile("" ::: "memory");
                    }
                    const float swk = ws[2][li][k], sak = ws[j][li][k];
                    const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : swk, lh ? 0.0f : sak, zf, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        y[j][e] = __builtin_fmaf(acc[e], S[e], y[j][e]);
                }
            if (k + 1 >= ng)                       // uniform
                break;
        }
    }

    // ---- the INT8 tail of the wave's blocks, in the waves of the first range
    if (T8 > 0 && ks == 0) {
        const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        const uint8_t *w8row = reinterpret_cast<const uint8_t *>(a.w8) + nrow * a.pitch8 + 16 * lh;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (j < nb) {
                const uint8_t *x8row = reinterpret_cast<const uint8_t *>(a.a8) + mrow[j] * a.pitch8 + 16 * lh;
                v16i acc8 = zi;
                for (int t = 0; t < T8; ++t) {
                    const v4i w0 = *reinterpret_cast<const v4i *>(w8row + t * kTileBytes);
                    const v4i w1 = *reinterpret_cast<const v4i *>(w8row + t * kTileBytes + 32);
                    const v4i x0 = *reinterpret_cast<const v4i *>(x8row + t * kTileBytes);
                    const v4i x1 = *reinterpret_cast<const v4i *>(x8row + t * kTileBytes + 32);
                    acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0, x0, acc8, 0, 0, 0);
                    acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1, x1, acc8, 0, 0, 0);
                }
                if constexpr (EXPORT) {
                    const int m = 32 * (b0 + j) + li;
                    if (m < a.M && a.acc8_out) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int n = n0 + 8 * (e / 4) + 4 * lh + e % 4;
                            if (n < a.N)
                                a.acc8_out[(int64_t)m * a.N + n] = acc8[e];
                        }
                    }
                }
                const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : a.sw8[nrow],
                                                                     lh ? 0.0f : a.sa8[mrow[j]], zf, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    y[j][e] = __builtin_fmaf((float)acc8[e], S[e], y[j][e]);
            }
    }

    // ---- partial blocks added in range order (deterministic), then Y
    __syncthreads();                               // every wave is done with the scale tables
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if (j < nb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                red[(((b0 + j) * KS + ks) * 16 + e) * 64 + lane] = y[j][e];
    __syncthreads();
    for (int i = tid; i < MB * 16 * 64 / 2; i += kDThreads) {
        const int l = i & 63, e0 = 2 * ((i >> 6) & 7), b = i >> 9;
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int r = 0; r < KS; ++r) {
            v0 += red[((b * KS + r) * 16 + e0) * 64 + l];
            v1 += red[((b * KS + r) * 16 + e0 + 1) * 64 + l];
        }
        const int m = 32 * b + (l & 31);
        const int n = n0 + 8 * (e0 / 4) + 4 * (l >> 5) + (e0 % 4);
        if (m < a.M) {
            _Float16 *dst = a.y + (int64_t)m * a.ldy + n;
            const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
            if (n + 1 < a.N && ((reinterpret_cast<uintptr_t>(dst) & 3) == 0)) {
                *reinterpret_cast<uint32_t *>(dst) =
                    (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            } else {
                if (n < a.N)
                    dst[0] = h0;
                if (n + 1 < a.N)
                    dst[1] = h1;
            }
        }
    }
}

}  // namespace gemm_fp6_impl

using namespace gemm_fp6_impl;

bool gemm_fp6_decode_fits(int32_t M, int32_t K_n, int32_t group) {
    const int G = K_n / 128, mb = (M + 31) / 32;
    if (mb == 5 || mb == 6 || mb == 7)               // 129..224 rows: the row-block counts with no instantiation
        return false;
    const int KS = kDWaves / ((mb + 1) / 2);          // group ranges
    const int gmax = mb > 4 ? 2 * kDMaxGroups : kDMaxGroups;
    return group == 128 && K_n % 128 == 0 && M > 32 && M <= 256 && (G + KS - 1) / KS <= gmax;
}

const char *gemm_fp6_decode_kernel_name(int32_t M) {
    switch ((M + 31) / 32) {
    case 2: return "gemm_fp6_decode_kernel<2, false>";
    case 3: return "gemm_fp6_decode_kernel<3, false>";
    case 4: return "gemm_fp6_decode_kernel<4, false>";
    default: return "gemm_fp6_decode_kernel<8, false>";
    }
}

hipError_t launch_gemm_fp6_decode(const Fp6GemmArgs &a, bool export_acc, hipStream_t stream) {
    const int blocks = (a.N + kDBN - 1) / kDBN;
    const int mb = (a.M + 31) / 32;
#define W4A4_FP6_DECODE(MBV)                                                                                     \
    if (export_acc)                                                                                              \
        hipLaunchKernelGGL((gemm_fp6_decode_kernel<MBV, true>), dim3(blocks), dim3(kDThreads), 0, stream, a);    \
    else                                                                                                         \
        hipLaunchKernelGGL((gemm_fp6_decode_kernel<MBV, false>), dim3(blocks), dim3(kDThreads), 0, stream, a);
    if (mb == 2) {
        W4A4_FP6_DECODE(2)
    } else if (mb == 3) {
        W4A4_FP6_DECODE(3)
    } else if (mb == 4) {
        W4A4_FP6_DECODE(4)
    } else {
        W4A4_FP6_DECODE(8)
    }
#undef W4A4_FP6_DECODE
    return hipGetLastError();
}

}  // namespace w4a4
