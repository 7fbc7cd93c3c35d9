// Streaming-read probe: how fast one GPU reads a buffer of a given size
// from HBM, for a given number of workgroups and loads in flight per lane.
// It is a measurement tool, not part of the layer: the decode GEMMs read
// their weights once, and this kernel gives the rate a plain read of the
// same bytes reaches with the same kind of loads (16 bytes per lane, the
// whole buffer split into contiguous ranges, one per workgroup).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads rounds [u0, u1) of the buffer; a round is DEPTH loads of
// 16 bytes per lane, each load of the wave covering 1 KB contiguous bytes and
// the DEPTH loads of a round issued before any is used.
template <int DEPTH, bool NT>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                              uint32_t *out) {
    const int64_t per = (int64_t)kThreads * DEPTH;
    const int64_t rounds = (n16 + per - 1) / per;
    const int64_t u0 = rounds * blockIdx.x / gridDim.x, u1 = rounds * (blockIdx.x + 1) / gridDim.x;
    uint32_t acc = 0;
    for (int64_t u = u0; u < u1; ++u) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t i = u * per + (int64_t)d * kThreads + threadIdx.x;
            if (i < n16)
                v[d] = NT ? __builtin_nontemporal_load(src + i) : src[i];
            else
                v[d] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    // the loads stay live: a store that the data decides on (out holds one
    // word per thread of the grid)
    if (acc == 0x9E3779B9u)
        out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int DEPTH>
hipError_t launch(const u32x4 *src, int64_t n16, int wgs, bool nt, uint32_t *out, hipStream_t stream) {
    if (nt)
        hipLaunchKernelGGL((read_probe_kernel<DEPTH, true>), dim3(wgs), dim3(kThreads), 0, stream, src, n16, out);
    else
        hipLaunchKernelGGL((read_probe_kernel<DEPTH, false>), dim3(wgs), dim3(kThreads), 0, stream, src, n16, out);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Words of `out` a launch with `wgs` workgroups may write (one per thread).
int64_t w4a4_read_probe_out_words(int32_t wgs) { return wgs > 0 ? (int64_t)wgs * kThreads : -1; }

// Read `bytes` (a multiple of 16) of device memory `src` (16-byte aligned)
// with `wgs` workgroups of 256 threads and `depth` (1, 2, 4, 8 or 16) loads
// of 16 bytes in flight per lane; `nontemporal` selects non-temporal loads.
// `out` is device memory of w4a4_read_probe_out_words(wgs) words, written
// only in the unlikely case that a lane's XOR of its data equals a fixed
// constant. Returns 0 on success, 1 for invalid arguments, 2 for a HIP error.
int32_t w4a4_read_probe(const void *src, int64_t bytes, int32_t wgs, int32_t depth, int32_t nontemporal,
                        void *out, void *stream) {
    if (!src || !out || bytes <= 0 || bytes % 16 != 0 || wgs <= 0 || (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    uint32_t *o = static_cast<uint32_t *>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n16 = bytes / 16;
    hipError_t err;
    switch (depth) {
    case 1: err = launch<1>(s, n16, wgs, nontemporal != 0, o, st); break;
    case 2: err = launch<2>(s, n16, wgs, nontemporal != 0, o, st); break;
    case 4: err = launch<4>(s, n16, wgs, nontemporal != 0, o, st); break;
    case 8: err = launch<8>(s, n16, wgs, nontemporal != 0, o, st); break;
    case 16: err = launch<16>(s, n16, wgs, nontemporal != 0, o, st); break;
    default: return 1;
    }
    return err == hipSuccess ? 0 : 2;
}

}  // extern "C"
