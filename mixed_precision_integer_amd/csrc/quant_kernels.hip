// Row quantizer for gfx950: gather by the outlier permutation, symmetric
// absmax scales, INT4 head (per row or per group) and INT8 tail, nibble pack.
//
// Method: QUIK abstract (4-bit operands, outlier channels kept in higher
// precision) and the Atom summary page (Summary paragraph 2: 8-bit outlier
// channels after reordering, group quantization, scales computed for every
// input at run time; Key points item 5: symmetric; Interesting ideas I1:
// outliers moved to a contiguous tail, I2: reordering fused into the
// quantizing pass).
//
// Design (HBM-bound: every input byte is read once, every code written once)
// * Persistent workgroups loop over rows. The permutation is read once per
//   workgroup into LDS as uint16; rows stream in by direct global->LDS DMA
//   (16 bytes per lane), double buffered: the next row's DMA is in flight
//   while the current row is quantized. LDS is sized statically per
//   row-length bucket (K <= 4096, 8192, 16384, 24576); long rows use more
//   lanes per workgroup so that each CU still runs 4 or more waves per SIMD.
// * A lane owns "units" of 8 reordered head channels (one packed dword of
//   output); consecutive lanes own consecutive units, so stores coalesce. A
//   unit's 8 fp16 values are gathered once and stay in registers as four
//   packed pairs for both passes (absmax in packed fp16, then codes).
// * Group absmax: groups are multiples of 128 channels = 16 units, so every
//   aligned 16-lane segment lies inside one group. Four xor-shuffles reduce a
//   segment and one lane folds it into the group's LDS maximum (float bits of
//   non-negative values order like unsigned integers). Per-row absmax and the
//   tail absmax are wave-shuffle + LDS reductions.
// * Code = rint(fl32(x / s)). Instead of one IEEE division per element the
//   kernel computes r = fl32(1 / s) once per block and the exact quotient by
//   Markstein's correction q0 = x r, e = fma(-q0, s, x), q1 = fma(e, r, q0),
//   which equals fl32(x / s) for every fp16 x and fp16 absmax; on that domain
//   |rint(q1)| <= qmax as well, so the clamp of the definition never fires
//   (both proved exhaustively by tests/test_exact_quotient.py). rint is
//   v_rndne_f32 (ties to even). Codes and scales are therefore bit-identical
//   to the definition. Offset codes q + 8 are packed with v_cvt_pk_u8_f32 and
//   turned into two's complement nibbles with one xor per dword.
#include <algorithm>

#include "w4a4_internal.h"

namespace w4a4 {
namespace quant_impl {

typedef _Float16 half2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float seg16_max(float v) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// fl32(x / s) from r = fl32(1 / s); r == 0 encodes s == 0 (then x == 0 too).
__device__ __forceinline__ float exact_quotient(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, r, q0);
}

__device__ __forceinline__ float recip_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

__device__ __forceinline__ _Float16 lo_half(uint32_t p) { return __builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFF)); }
__device__ __forceinline__ _Float16 hi_half(uint32_t p) { return __builtin_bit_cast(_Float16, (uint16_t)(p >> 16)); }

// s_waitcnt immediates (gfx9 encoding): all counters zero, or LDS only.
constexpr int kWaitAll = 0;
constexpr int kWaitLds = 0xF | (0x3 << 14) | (0x7 << 4);   // vmcnt max, expcnt max, lgkmcnt 0

// Workgroup barrier that orders LDS traffic only: in-flight row DMA (vmcnt)
// keeps running across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLds);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Static LDS for rows of up to KMAX channels: the permutation as uint16, two
// row buffers (whole DMA rounds) and the group tables.
template <int KMAX, int THREADS>
struct RowLds {
    static constexpr int ROUND = THREADS * 16;   // bytes one DMA instruction moves per workgroup
    static constexpr int XB = (KMAX * 2 + ROUND - 1) / ROUND * ROUND;
    static constexpr int GMAX = KMAX / 128;
    uint16_t perm[KMAX];
    unsigned char x[2][XB];
    float gs[GMAX], gr[GMAX];
    unsigned gmax[2][GMAX];
};

template <int KMAX, int THREADS, bool GROUPED>
__global__ __launch_bounds__(THREADS) void quant_rows_kernel(QuantArgs a) {
    using L = RowLds<KMAX, THREADS>;
    constexpr int GMAX = L::GMAX, NW = THREADS / 64;
    constexpr int UMAX = (KMAX / 8 + THREADS - 1) / THREADS;   // head units per lane
    __shared__ __align__(16) L sm;
    __shared__ float red_h[NW], red_t[NW], row_sr[4];

    const int K = a.K, K_n = a.K_n, n_out = a.n_out, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint16_t *perm16 = sm.perm;
    unsigned *gmax = &sm.gmax[0][0];

    const int nfull = K / 8;                       // whole 16-byte chunks of a row
    const int rounds = (nfull + THREADS - 1) / THREADS;
    auto issue_row = [&](int row, int b) {
        const unsigned char *src = reinterpret_cast<const unsigned char *>(a.src + (int64_t)row * a.ld);
        const uint32_t d = lds_addr(sm.x[b]) + wave_u * 1024;
        for (int j = 0; j < rounds; ++j) {
            const int c = j * THREADS + tid;
            dma16(src, (uint32_t)(c < nfull ? c : 0) * 16, d + j * L::ROUND);
        }
    };

    const int U = (K_n + 7) / 8;
    const int W4 = (int)(a.pitch4 / 4), W8 = (int)(a.pitch8 / 4);

    int row = blockIdx.x;
    if (row < a.rows)
        issue_row(row, 0);
    // permutation -> LDS (uint16), once per workgroup, while the first row streams in
    for (int j = tid; j < K; j += THREADS)
        perm16[j] = (uint16_t)a.perm[j];
    if (GROUPED)
        for (int t = tid; t < 2 * GMAX; t += THREADS)
            gmax[t] = 0u;
    for (int it = 0; row < a.rows; ++it, row += gridDim.x) {
        const int buf = it & 1;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(sm.x[buf]);
        unsigned *gm = gmax + buf * GMAX;
        // (1) this row has landed in LDS and the previous row is finished
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (K % 8) {                               // ragged row end: plain loads, before
            const _Float16 *src = a.src + (int64_t)row * a.ld;   // the next row's DMA
            if (tid < K % 8)
                reinterpret_cast<_Float16 *>(sm.x[buf])[nfull * 8 + tid] = src[nfull * 8 + tid];
            lds_barrier();
        }
        if (row + (int)gridDim.x < a.rows)
            issue_row(row + gridDim.x, buf ^ 1);

        // (2) gather the head units into registers; absmax in packed fp16
        uint32_t v[UMAX][4];
        float hmax = 0.0f, tmax = 0.0f;
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = i * THREADS + tid;
            const int j0 = u * 8;
            if (u < U && j0 + 8 <= K_n) {
                const uint4 p = *reinterpret_cast<const uint4 *>(perm16 + j0);
                const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[i][k] = (uint32_t)xs[w[k] & 0xFFFF] | ((uint32_t)xs[w[k] >> 16] << 16);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = j0 + 2 * k;
                    const uint32_t lo = (u < U && j < K_n) ? xs[perm16[j]] : 0u;
                    const uint32_t hi = (u < U && j + 1 < K_n) ? xs[perm16[j + 1]] : 0u;
                    v[i][k] = lo | (hi << 16);
                }
            }
            half2 m2 = {(_Float16)0, (_Float16)0};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(half2, v[i][k] & 0x7FFF7FFFu));
            float m = fmaxf((float)m2.x, (float)m2.y);
            if (GROUPED) {
                if (i * THREADS < U) {             // uniform: every lane of the wave takes part
                    m = seg16_max(m);
                    if ((lane & 15) == 0 && u < U)
                        atomicMax(&gm[j0 / a.group], __float_as_uint(m));
                }
            } else {
                hmax = fmaxf(hmax, m);
            }
        }
        for (int j = K_n + tid; j < K; j += THREADS)
            tmax = fmaxf(tmax, fabsf((float)__builtin_bit_cast(_Float16, xs[perm16[j]])));
        hmax = wave_max(hmax);
        tmax = wave_max(tmax);
        if (lane == 0) {
            red_h[wave] = hmax;
            red_t[wave] = tmax;
        }
        lds_barrier();

        // (3) scales and reciprocals
        if (GROUPED) {
            for (int t = tid; t < G; t += THREADS) {
                const float s = __uint_as_float(gm[t]) / 7.0f;
                sm.gs[t] = s;
                sm.gr[t] = recip_or_zero(s);
                a.s4[(int64_t)row * G + t] = s;
                gmax[(buf ^ 1) * GMAX + t] = 0u;   // the next row accumulates there
            }
        }
        if (tid == 0) {
            float ra = 0.0f, ta = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                ra = fmaxf(ra, red_h[w]);
                ta = fmaxf(ta, red_t[w]);
            }
            const float s = ra / 7.0f, s8 = ta / 127.0f;
            row_sr[0] = s;
            row_sr[1] = recip_or_zero(s);
            row_sr[2] = s8;
            row_sr[3] = recip_or_zero(s8);
            if (!GROUPED && G > 0)
                a.s4[row] = s;
            if (a.s8)
                a.s8[row] = n_out > 0 ? s8 : 0.0f;
        }
        lds_barrier();

        // (4) INT4 head: codes + 8 as bytes, even channels in one dword and odd
        //     ones in another, then one nibble interleave and an xor with 8
        uint32_t *q4row = reinterpret_cast<uint32_t *>(a.q4 + (int64_t)row * a.pitch4);
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = i * THREADS + tid;
            if (u < U) {
                float s, r;
                if (GROUPED) {
                    const int t = (u * 8) / a.group;
                    s = sm.gs[t];
                    r = sm.gr[t];
                } else {
                    s = row_sr[0];
                    r = row_sr[1];
                }
                uint32_t ev = 0, od = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float c0 = __builtin_rintf(exact_quotient((float)lo_half(v[i][k]), s, r)) + 8.0f;
                    const float c1 = __builtin_rintf(exact_quotient((float)hi_half(v[i][k]), s, r)) + 8.0f;
                    ev = __builtin_amdgcn_cvt_pk_u8_f32(c0, k, ev);
                    od = __builtin_amdgcn_cvt_pk_u8_f32(c1, k, od);
                }
                q4row[u] = (ev | (od << 4)) ^ 0x88888888u;
            }
        }
        for (int u = U + tid; u < W4; u += THREADS)   // zero padding of the row pitch
            q4row[u] = 0u;

        // (5) INT8 tail: 4 codes -> one dword
        if (a.q8) {
            uint32_t *q8row = reinterpret_cast<uint32_t *>(a.q8 + (int64_t)row * a.pitch8);
            const float s8 = row_sr[2], r8 = row_sr[3];
            for (int w = tid; w < W8; w += THREADS) {
                uint32_t word = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = K_n + w * 4 + k;
                    if (j < K) {
                        const float x = (float)__builtin_bit_cast(_Float16, xs[perm16[j]]);
                        const int q = (int)__builtin_rintf(exact_quotient(x, s8, r8));
                        word |= (uint32_t)(q & 0xFF) << (8 * k);
                    }
                }
                q8row[w] = word;
            }
        }
    }
}

template <int KMAX, int THREADS, bool GROUPED>
hipError_t launch(const QuantArgs &a, hipStream_t stream) {
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_kernel<KMAX, THREADS, GROUPED>,
                                                     THREADS, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int grid = (int)std::min<long>(a.rows, (long)cus * per_cu);
    hipLaunchKernelGGL((quant_rows_kernel<KMAX, THREADS, GROUPED>), dim3(grid), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

// Row-length buckets: (longest row, lanes per workgroup).
template <bool GROUPED>
hipError_t launch_grouping(const QuantArgs &a, hipStream_t stream) {
    if (a.K <= 4096) return launch<4096, 256, GROUPED>(a, stream);
    if (a.K <= 8192) return launch<8192, 512, GROUPED>(a, stream);
    if (a.K <= 16384) return launch<16384, 1024, GROUPED>(a, stream);
    if (a.K <= 24576) return launch<24576, 1024, GROUPED>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace quant_impl

int quant_rows_max_k() { return 24576; }

hipError_t launch_quant_rows(const QuantArgs &a, hipStream_t stream) {
    if (a.rows == 0)
        return hipSuccess;
    return a.group > 0 ? quant_impl::launch_grouping<true>(a, stream)
                       : quant_impl::launch_grouping<false>(a, stream);
}

}  // namespace w4a4
