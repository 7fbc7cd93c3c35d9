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
// One workgroup (256 lanes, 4 wave64) per row. The row is streamed from HBM
// once with 16-byte coalesced loads into LDS; the permutation gather then
// reads LDS only. Each lane owns "units" of 8 reordered head channels (one
// packed dword of output) or 4 tail channels (one int8 dword). Per-unit
// absmax values are reduced with wave shuffles (per-row scales) or through a
// small LDS table (group scales). The division x / s is the correctly rounded
// IEEE fp32 division and rint is v_rndne_f32 (ties to even), so codes and
// scales are bit-identical to any other IEEE implementation of the same
// definition.
#include "w4a4_internal.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Symmetric code: q = clamp(rint(x / s), lo, hi); s == 0 gives 0.
__device__ __forceinline__ int quant_code(float x, float s, float lo, float hi) {
    if (s == 0.0f)
        return 0;
    float r = __builtin_rintf(x / s);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

template <bool GROUPED>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(QuantArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int K = a.K, K_n = a.K_n, n_out = a.n_out;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // LDS carve-up: fp16 row (rounded to 16 B), unit maxima, group scales.
    const int kpad = (K + 7) & ~7;
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    const int U = (K_n + 7) / 8;                 // head units of 8 channels
    float *umax = reinterpret_cast<float *>(smem + kpad * 2);
    float *gscale = umax + (GROUPED ? U : 0);
    __shared__ float red_h[4], red_t[4];

    // 1. stream the row into LDS (16-byte loads, coalesced)
    const _Float16 *src = a.src + (int64_t)row * a.ld;
    const int nvec = K / 8;
    for (int c = tid; c < nvec; c += kThreads)
        reinterpret_cast<uint4 *>(xs)[c] = reinterpret_cast<const uint4 *>(src)[c];
    for (int j = nvec * 8 + tid; j < K; j += kThreads)
        xs[j] = src[j];
    __syncthreads();

    // 2. absmax: per head unit, and over the tail
    float hmax = 0.0f, tmax = 0.0f;
    for (int u = tid; u < U; u += kThreads) {
        const int j0 = u * 8;
        float m = 0.0f;
        if (j0 + 8 <= K_n) {
            const int4 p0 = reinterpret_cast<const int4 *>(a.perm + j0)[0];
            const int4 p1 = reinterpret_cast<const int4 *>(a.perm + j0)[1];
            const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k)
                m = fmaxf(m, fabsf((float)xs[idx[k]]));
        } else {
            for (int j = j0; j < K_n; ++j)
                m = fmaxf(m, fabsf((float)xs[a.perm[j]]));
        }
        if (GROUPED)
            umax[u] = m;
        else
            hmax = fmaxf(hmax, m);
    }
    const int UT = (n_out + 3) / 4;              // tail units of 4 channels
    for (int v = tid; v < UT; v += kThreads) {
        for (int j = K_n + v * 4; j < K_n + v * 4 + 4 && j < K; ++j)
            tmax = fmaxf(tmax, fabsf((float)xs[a.perm[j]]));
    }
    hmax = wave_max(hmax);
    tmax = wave_max(tmax);
    if (lane == 0) {
        red_h[wave] = hmax;
        red_t[wave] = tmax;
    }
    __syncthreads();
    const float row_amax = fmaxf(fmaxf(red_h[0], red_h[1]), fmaxf(red_h[2], red_h[3]));
    const float tail_amax = fmaxf(fmaxf(red_t[0], red_t[1]), fmaxf(red_t[2], red_t[3]));

    // 3. scales
    float s_row = 0.0f;
    if (GROUPED) {
        const int upg = a.group / 8;             // units per group
        for (int t = tid; t < a.G; t += kThreads) {
            float m = 0.0f;
            for (int u = t * upg; u < (t + 1) * upg; ++u)
                m = fmaxf(m, umax[u]);
            const float s = m / 7.0f;
            gscale[t] = s;
            a.s4[(int64_t)row * a.G + t] = s;
        }
        __syncthreads();
    } else {
        s_row = row_amax / 7.0f;
        if (tid == 0 && a.G > 0)
            a.s4[row] = s_row;
    }
    const float s_tail = tail_amax / 127.0f;
    if (tid == 0 && a.s8)
        a.s8[row] = n_out > 0 ? s_tail : 0.0f;

    // 4. INT4 head: 8 codes -> one packed dword, low nibble first
    uint32_t *q4row = reinterpret_cast<uint32_t *>(a.q4 + (int64_t)row * a.pitch4);
    const int W4 = (int)(a.pitch4 / 4);
    for (int u = tid; u < W4; u += kThreads) {
        uint32_t word = 0;
        if (u < U) {
            const float s = GROUPED ? gscale[(u * 8) / a.group] : s_row;
            const int j0 = u * 8;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = j0 + k;
                if (j < K_n) {
                    const int q = quant_code((float)xs[a.perm[j]], s, -8.0f, 7.0f);
                    word |= (uint32_t)(q & 0xF) << (4 * k);
                }
            }
        }
        q4row[u] = word;
    }

    // 5. INT8 tail: 4 codes -> one dword
    if (a.q8) {
        uint32_t *q8row = reinterpret_cast<uint32_t *>(a.q8 + (int64_t)row * a.pitch8);
        const int W8 = (int)(a.pitch8 / 4);
        for (int v = tid; v < W8; v += kThreads) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = K_n + v * 4 + k;
                if (j < K) {
                    const int q = quant_code((float)xs[a.perm[j]], s_tail, -128.0f, 127.0f);
                    word |= (uint32_t)(q & 0xFF) << (8 * k);
                }
            }
            q8row[v] = word;
        }
    }
}

}  // namespace

hipError_t launch_quant_rows(const QuantArgs &a, hipStream_t stream) {
    if (a.rows == 0)
        return hipSuccess;
    const int kpad = (a.K + 7) & ~7;
    const int U = (a.K_n + 7) / 8;
    const bool grouped = a.group > 0;
    const size_t lds = (size_t)kpad * 2 + (grouped ? (size_t)(U + a.G) * 4 : 0);
    if (grouped)
        hipLaunchKernelGGL(quant_rows_kernel<true>, dim3(a.rows), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(quant_rows_kernel<false>, dim3(a.rows), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
