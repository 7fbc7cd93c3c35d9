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
// * A lane takes 8 channels of one head vector with one 16-byte access; a
//   head vector is an aligned segment of D / 8 lanes (8, 16 or 32), so one
//   wave instruction covers 512 channels (8, 4 or 2 head vectors) and the
//   head's absmax is a few xor-shuffles inside its segment. Each wave works
//   through kSteps such groups, with all their loads issued before the first
//   is reduced.
// * Codes by the exact quotient the row quantizer uses (r = fl32(1 / s),
//   q0 = x r, e = fma(-q0, s, x), q = fma(e, r, q0): the correctly rounded x / s
//   for every fp16 x and every reachable scale, with |rint(q)| <= qmax, both
//   checked exhaustively), so the codes match the definition bit for bit.
//   Offset codes are packed to bytes with v_cvt_pk_u8_f32; INT4 codes are
//   interleaved two per byte, low nibble first (the layer's packing), and
//   turned back to two's complement with one xor per dword.
// * The new tokens' fp16 vectors are read once and the INT4 codes written
//   once, so both use non-temporal accesses (streamed past the caches): the
//   quantizing store measured 18-20% faster with them. The gather keeps plain
//   accesses, which measured faster there.
// * The slot mapping gives each token's cache slot; a slot outside
//   [0, num_slots) is skipped when quantizing and reads as zeros when
//   gathering, so a bad slot cannot write outside the cache.
#include "quant_internal.h"

namespace w4a4 {
namespace kv_impl {

constexpr int kSteps = 4;           // 512-channel groups per wave

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exact_quotient(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, r, q0);
}

__device__ __forceinline__ float lo_f(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFF)); }
__device__ __forceinline__ float hi_f(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16)); }

// SEG = D / 8 lanes per head vector; HPW = 64 / SEG head vectors per step.
template <int SEG, int BITS>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t *X, int64_t ldx, int T, int H,
                                                       const int32_t *slots, int64_t num_slots, uint8_t *cq,
                                                       float *cs) {
    constexpr int D = 8 * SEG, HPW = 64 / SEG;
    constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
    constexpr int VB = D * BITS / 8;                 // cache bytes per head vector
    const int lane = threadIdx.x & 63, part = lane % SEG, g = lane / SEG;
    const int64_t nvec = (int64_t)T * H;
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kSteps * HPW;
    uint4 x[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int64_t v = min(base + i * HPW + g, nvec - 1);   // clamped: every load in bounds
        const int64_t t = v / H, h = v % H;
        const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(X + t * ldx + h * D + part * 8));
        x[i] = uint4{q.x, q.y, q.z, q.w};
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if (base + i * HPW >= nvec)
            break;                                   // uniform over the wave
        const int64_t v = base + i * HPW + g;
        const int64_t t = min(v, nvec - 1) / H, h = min(v, nvec - 1) % H;
        const int64_t slot = slots ? (int64_t)slots[t] : t;
        const bool live = v < nvec && slot >= 0 && slot < num_slots;
        const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = fmaxf(m, fmaxf(fabsf(lo_f(w[k])), fabsf(hi_f(w[k]))));
#pragma unroll
        for (int off = 1; off < SEG; off <<= 1)      // segment max (all lanes take part)
            m = fmaxf(m, __shfl_xor(m, off, 64));
        const float s = m / qmax, r = s == 0.0f ? 0.0f : 1.0f / s;
        if (!live)
            continue;
        uint8_t *dst = cq + (slot * H + h) * VB;
        if constexpr (BITS == 4) {
            uint32_t ev = 0, od = 0;                 // offset codes of the even / odd channels
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(lo_f(w[k]), s, r)) + 8.0f, k, ev);
                od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(hi_f(w[k]), s, r)) + 8.0f, k, od);
            }
            __builtin_nontemporal_store((ev | (od << 4)) ^ 0x88888888u, reinterpret_cast<uint32_t *>(dst) + part);
        } else {
            uint32_t b0 = 0, b1 = 0;                 // channels 0-3 and 4-7, offset by 128
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                b0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(lo_f(w[k]), s, r)) + 128.0f, 2 * k, b0);
                b0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(hi_f(w[k]), s, r)) + 128.0f, 2 * k + 1, b0);
                b1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(lo_f(w[k + 2]), s, r)) + 128.0f, 2 * k, b1);
                b1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(hi_f(w[k + 2]), s, r)) + 128.0f, 2 * k + 1, b1);
            }
            reinterpret_cast<uint2 *>(dst)[part] = uint2{b0 ^ 0x80808080u, b1 ^ 0x80808080u};
        }
        if (part == 0)
            cs[slot * H + h] = s;
    }
}

template <int SEG, int BITS>
__global__ __launch_bounds__(256) void kv_dequant_kernel(const uint8_t *cq, const float *cs, int64_t num_slots,
                                                         const int32_t *slots, int T, int H, uint16_t *Y,
                                                         int64_t ldy) {
#pragma clang fp contract(off)
    constexpr int D = 8 * SEG, HPW = 64 / SEG;
    constexpr int VB = D * BITS / 8;
    const int lane = threadIdx.x & 63, part = lane % SEG, g = lane / SEG;
    const int64_t nvec = (int64_t)T * H;
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kSteps * HPW;
    uint2 c[kSteps];
    float sc[kSteps];
    bool ok[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int64_t v = min(base + i * HPW + g, nvec - 1);
        const int64_t t = v / H, h = v % H;
        int64_t slot = slots ? (int64_t)slots[t] : t;
        ok[i] = slot >= 0 && slot < num_slots;
        slot = ok[i] ? slot : 0;                     // in-bounds address, value discarded
        const uint8_t *src = cq + (slot * H + h) * VB;
        if constexpr (BITS == 4)
            c[i] = uint2{reinterpret_cast<const uint32_t *>(src)[part], 0u};
        else
            c[i] = reinterpret_cast<const uint2 *>(src)[part];
        sc[i] = cs[slot * H + h];
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int64_t v = base + i * HPW + g;
        if (base + i * HPW >= nvec)
            break;
        if (v >= nvec)
            continue;
        int q[8];
        if constexpr (BITS == 4) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                q[k] = (int)(((c[i].x >> (4 * k)) & 0xF) ^ 8) - 8;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                q[k] = (int)(int8_t)(((k < 4 ? c[i].x : c[i].y) >> (8 * (k & 3))) & 0xFF);
        }
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const _Float16 a = ok[i] ? (_Float16)(sc[i] * (float)q[2 * k]) : (_Float16)0.0f;
            const _Float16 b = ok[i] ? (_Float16)(sc[i] * (float)q[2 * k + 1]) : (_Float16)0.0f;
            o[k] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
        }
        const int64_t t = v / H, h = v % H;
        *reinterpret_cast<uint4 *>(Y + t * ldy + h * D + part * 8) = uint4{o[0], o[1], o[2], o[3]};
    }
}

// fp16 data passes to the kernels as its bit patterns (uint16_t), so that
// kernel names in traces demangle.
inline const uint16_t *fp16_bits(const _Float16 *p) { return reinterpret_cast<const uint16_t *>(p); }

template <int SEG>
hipError_t launch_seg(const KvArgs &a, bool quant, hipStream_t stream) {
    constexpr int HPW = 64 / SEG;
    const int64_t nvec = (int64_t)a.T * a.H;
    const int64_t per_group = 4LL * kSteps * HPW;
    const int grid = (int)((nvec + per_group - 1) / per_group);
    if (quant) {
        if (a.bits == 4)
            hipLaunchKernelGGL((kv_quant_kernel<SEG, 4>), dim3(grid), dim3(256), 0, stream, fp16_bits(a.X), a.ldx, a.T, a.H,
                               a.slots, a.num_slots, a.cq, a.cs);
        else
            hipLaunchKernelGGL((kv_quant_kernel<SEG, 8>), dim3(grid), dim3(256), 0, stream, fp16_bits(a.X), a.ldx, a.T, a.H,
                               a.slots, a.num_slots, a.cq, a.cs);
    } else {
        if (a.bits == 4)
            hipLaunchKernelGGL((kv_dequant_kernel<SEG, 4>), dim3(grid), dim3(256), 0, stream, a.cq, a.cs,
                               a.num_slots, a.slots, a.T, a.H, reinterpret_cast<uint16_t *>(a.Y), a.ldy);
        else
            hipLaunchKernelGGL((kv_dequant_kernel<SEG, 8>), dim3(grid), dim3(256), 0, stream, a.cq, a.cs,
                               a.num_slots, a.slots, a.T, a.H, reinterpret_cast<uint16_t *>(a.Y), a.ldy);
    }
    return hipGetLastError();
}

}  // namespace kv_impl

hipError_t launch_kv(const KvArgs &a, bool quant, hipStream_t stream) {
    if (a.T == 0 || a.H == 0)
        return hipSuccess;
    switch (a.D) {
    case 64: return kv_impl::launch_seg<8>(a, quant, stream);
    case 128: return kv_impl::launch_seg<16>(a, quant, stream);
    case 256: return kv_impl::launch_seg<32>(a, quant, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a4
