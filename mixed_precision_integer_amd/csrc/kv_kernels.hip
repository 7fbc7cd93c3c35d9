// Low-bit KV cache for gfx950: quantize the key or value vectors of new
// tokens into a slot-mapped cache (INT4 or INT8, one fp32 scale per token and
// head), and gather them back to fp16.
//
// Method: the Atom summary page keeps the KV cache in low bit-width (Summary
// paragraph 2); the NQKV abstract on the "smoothquant" tag page quantizes the
// cache block by block. Each (token, head) vector of D channels is one block
// of the layer's symmetric quantizer: s = fl32(absmax / qmax), q = rint of
// the correctly rounded quotient x / s (qmax 7 or 127); dequantization is
// fp16(fl32(s * q)).
//
// Design (HBM-bound: every input byte read once, every code written once)
// * One wave per head vector at a time: lane l holds channels E l .. E l + E - 1
//   (E = D / 64), so a wave reads D * 2 contiguous bytes; the absmax is a wave
//   max. Each wave takes kVecs consecutive vectors and issues all their loads
//   before it reduces the first, so eight loads per lane are in flight.
// * Codes by the exact quotient the row quantizer uses (r = fl32(1 / s),
//   q0 = x r, e = fma(-q0, s, x), q = fma(e, r, q0): the correctly rounded x / s
//   for every fp16 x and every reachable scale, with |rint(q)| <= qmax, both
//   checked exhaustively), so the codes match the definition bit for bit.
// * INT4 codes are packed two per byte, low nibble first (the layer's
//   packing); for D = 64 two neighbouring lanes combine their nibbles.
// * The slot mapping gives each token's cache slot; a slot outside
//   [0, num_slots) is skipped when quantizing and reads as zeros when
//   gathering, so a bad slot cannot write outside the cache.
#include "quant_internal.h"

namespace w4a4 {
namespace kv_impl {

constexpr int kVecs = 8;            // head vectors per wave

__device__ __forceinline__ float exact_quotient(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, r, q0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

template <int E>
struct Halves {
    _Float16 h[E];
};

template <int E>
__device__ __forceinline__ Halves<E> load_halves(const _Float16 *p) {
    Halves<E> r;
    if constexpr (E == 1) {
        r.h[0] = *p;
    } else if constexpr (E == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
        r.h[0] = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF));
        r.h[1] = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        r.h[0] = __builtin_bit_cast(_Float16, (uint16_t)(w.x & 0xFFFF));
        r.h[1] = __builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16));
        r.h[2] = __builtin_bit_cast(_Float16, (uint16_t)(w.y & 0xFFFF));
        r.h[3] = __builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16));
    }
    return r;
}

template <int E, int BITS>
__global__ __launch_bounds__(256) void kv_quant_kernel(const _Float16 *X, int64_t ldx, int T, int H,
                                                       const int32_t *slots, int64_t num_slots, uint8_t *cq,
                                                       float *cs) {
    constexpr int D = 64 * E;
    constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
    constexpr int VB = D * BITS / 8;                 // cache bytes per head vector
    const int lane = threadIdx.x & 63;
    const int64_t nvec = (int64_t)T * H;
    const int64_t v0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kVecs;
    Halves<E> x[kVecs];
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        const int64_t v = min(v0 + i, nvec - 1);     // clamped: every load in bounds
        const int64_t t = v / H, h = v % H;
        x[i] = load_halves<E>(X + t * ldx + h * D + lane * E);
    }
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        const int64_t v = v0 + i;
        if (v >= nvec)
            break;                                   // uniform over the wave
        const int64_t t = v / H, h = v % H;
        const int64_t slot = slots ? (int64_t)slots[t] : t;
        if (slot < 0 || slot >= num_slots)
            continue;                                // uniform over the wave
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            m = fmaxf(m, fabsf((float)x[i].h[e]));
        m = wave_max(m);
        const float s = m / qmax, r = s == 0.0f ? 0.0f : 1.0f / s;
        int q[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            q[e] = (int)__builtin_rintf(exact_quotient((float)x[i].h[e], s, r));
        uint8_t *dst = cq + (slot * H + h) * VB;
        if constexpr (BITS == 8) {
            if constexpr (E == 1) {
                dst[lane] = (uint8_t)q[0];
            } else if constexpr (E == 2) {
                reinterpret_cast<uint16_t *>(dst)[lane] = (uint16_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8));
            } else {
                reinterpret_cast<uint32_t *>(dst)[lane] = (uint32_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8) |
                                                                     ((q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24));
            }
        } else {
            if constexpr (E == 1) {
                const int nxt = __shfl_down(q[0], 1, 64);
                if ((lane & 1) == 0)
                    dst[lane >> 1] = (uint8_t)((q[0] & 0xF) | ((nxt & 0xF) << 4));
            } else if constexpr (E == 2) {
                dst[lane] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
            } else {
                reinterpret_cast<uint16_t *>(dst)[lane] =
                    (uint16_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4) | ((q[2] & 0xF) << 8) | ((q[3] & 0xF) << 12));
            }
        }
        if (lane == 0)
            cs[slot * H + h] = s;
    }
}

template <int E, int BITS>
__global__ __launch_bounds__(256) void kv_dequant_kernel(const uint8_t *cq, const float *cs, int64_t num_slots,
                                                         const int32_t *slots, int T, int H, _Float16 *Y,
                                                         int64_t ldy) {
#pragma clang fp contract(off)
    constexpr int D = 64 * E;
    constexpr int VB = D * BITS / 8;
    const int lane = threadIdx.x & 63;
    const int64_t nvec = (int64_t)T * H;
    const int64_t v0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kVecs;
    int q[kVecs][E];
    float sc[kVecs];
    bool okv[kVecs];
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        const int64_t v = min(v0 + i, nvec - 1);
        const int64_t t = v / H, h = v % H;
        int64_t slot = slots ? (int64_t)slots[t] : t;
        const bool ok = slot >= 0 && slot < num_slots;
        slot = ok ? slot : 0;                        // in-bounds address, value discarded
        const uint8_t *src = cq + (slot * H + h) * VB;
        sc[i] = cs[slot * H + h];
        okv[i] = ok;
        if constexpr (BITS == 8) {
            if constexpr (E == 1) {
                q[i][0] = (int8_t)src[lane];
            } else if constexpr (E == 2) {
                const uint16_t w = reinterpret_cast<const uint16_t *>(src)[lane];
                q[i][0] = (int8_t)(w & 0xFF);
                q[i][1] = (int8_t)(w >> 8);
            } else {
                const uint32_t w = reinterpret_cast<const uint32_t *>(src)[lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    q[i][e] = (int8_t)((w >> (8 * e)) & 0xFF);
            }
        } else {
            if constexpr (E == 1) {
                const uint8_t b = src[lane >> 1];
                const int nib = (lane & 1) ? (b >> 4) : (b & 0xF);
                q[i][0] = (nib ^ 8) - 8;
            } else if constexpr (E == 2) {
                const uint8_t b = src[lane];
                q[i][0] = ((b & 0xF) ^ 8) - 8;
                q[i][1] = ((b >> 4) ^ 8) - 8;
            } else {
                const uint16_t w = reinterpret_cast<const uint16_t *>(src)[lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    q[i][e] = (((w >> (4 * e)) & 0xF) ^ 8) - 8;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        const int64_t v = v0 + i;
        if (v >= nvec)
            break;
        const int64_t t = v / H, h = v % H;
        _Float16 *dst = Y + t * ldy + h * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e)
            dst[e] = okv[i] ? (_Float16)(sc[i] * (float)q[i][e]) : (_Float16)0.0f;
    }
}

template <int E>
hipError_t launch_e(const KvArgs &a, bool quant, hipStream_t stream) {
    const int64_t nvec = (int64_t)a.T * a.H;
    const int grid = (int)((nvec + 4 * kVecs - 1) / (4 * kVecs));
    if (quant) {
        if (a.bits == 4)
            hipLaunchKernelGGL((kv_quant_kernel<E, 4>), dim3(grid), dim3(256), 0, stream, a.X, a.ldx, a.T, a.H,
                               a.slots, a.num_slots, a.cq, a.cs);
        else
            hipLaunchKernelGGL((kv_quant_kernel<E, 8>), dim3(grid), dim3(256), 0, stream, a.X, a.ldx, a.T, a.H,
                               a.slots, a.num_slots, a.cq, a.cs);
    } else {
        if (a.bits == 4)
            hipLaunchKernelGGL((kv_dequant_kernel<E, 4>), dim3(grid), dim3(256), 0, stream, a.cq, a.cs,
                               a.num_slots, a.slots, a.T, a.H, a.Y, a.ldy);
        else
            hipLaunchKernelGGL((kv_dequant_kernel<E, 8>), dim3(grid), dim3(256), 0, stream, a.cq, a.cs,
                               a.num_slots, a.slots, a.T, a.H, a.Y, a.ldy);
    }
    return hipGetLastError();
}

}  // namespace kv_impl

hipError_t launch_kv(const KvArgs &a, bool quant, hipStream_t stream) {
    if (a.T == 0 || a.H == 0)
        return hipSuccess;
    switch (a.D) {
    case 64: return kv_impl::launch_e<1>(a, quant, stream);
    case 128: return kv_impl::launch_e<2>(a, quant, stream);
    case 256: return kv_impl::launch_e<4>(a, quant, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a4
