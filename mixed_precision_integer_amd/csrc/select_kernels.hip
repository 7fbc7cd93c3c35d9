// Offline outlier-channel selection for gfx950: the n_out channels with the
// largest absolute value over a calibration batch, ties to the lower channel
// index, written ascending, together with the layer's permutation (the other
// channels ascending, then the selected ones).
//
// Method: the Atom summary page keeps a small set of outlier channels in 8
// bits after reordering them to a contiguous tail (Summary paragraph 2,
// Interesting ideas I1 and I3); the QUIK abstract keeps some outlier
// activations in higher precision. Neither page gives the rule that picks
// the channels; the score here is the per-channel absmax, the statistic the
// quantizer itself scales by.
//
// Design
// * Column absmax (HBM-bound: the batch is read once). A workgroup owns a
//   stripe of 512 columns (64 lanes x 8 fp16 = one 16-byte load per lane and
//   row, 1 KB per wave instruction) and a chunk of rows; its four waves take
//   every fourth row, four rows in flight per lane. Magnitudes are compared
//   as the fp16 bit patterns with the sign cleared (for finite values they
//   order like the values), two per dword with packed 16-bit max. The waves
//   meet in LDS and the chunk's maxima go to a partial row in the workspace.
// * A second launch folds the chunk partials into one key per channel.
// * Selection in one workgroup of 1024 lanes, the keys in LDS. A two-level
//   radix select (high byte, then low byte among keys in the chosen high
//   bin) finds the threshold key T and how many keys equal to T are taken;
//   two block-wide scans over channels in index order then apply the
//   lower-index rule and give every channel its output position.
#include <algorithm>

#include "quant_internal.h"

namespace w4a4 {
namespace select_impl {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kStripe = 512;          // columns per workgroup
constexpr int kWaves = 4;             // waves per column-absmax workgroup
constexpr int kRowsInFlight = 4;      // rows each lane loads before it reduces
constexpr int kTargetGroups = 2048;   // column-absmax workgroups: 8 resident per CU
constexpr int kMinRowsPerChunk = 16;
constexpr int kMaxK = 32768;          // keys held in LDS by the select launch
constexpr int kSelThreads = 1024;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                                                  __builtin_bit_cast(ushort2_t, b)));
}

__global__ __launch_bounds__(kWaves * 64) void colmax_kernel(const uint16_t *X, int64_t ld, int rows, int K,
                                                             int rows_per_chunk, int64_t kp, uint16_t *partial) {
    __shared__ uint4 red[kWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * kStripe + lane * 8;
    const int r0 = blockIdx.y * rows_per_chunk;
    const int r1 = min(r0 + rows_per_chunk, rows);
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    if (c0 + 8 <= K) {
        for (int r = r0 + wave; r < r1; r += kWaves * kRowsInFlight) {
            uint4 v[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                const int rr = r + u * kWaves;
                if (rr < r1) {                           // each value is read once: streamed past the caches
                    const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(X + (int64_t)rr * ld + c0));
                    v[u] = uint4{q.x, q.y, q.z, q.w};
                } else {
                    v[u] = uint4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                m[0] = max_u16x2(m[0], v[u].x & 0x7FFF7FFFu);
                m[1] = max_u16x2(m[1], v[u].y & 0x7FFF7FFFu);
                m[2] = max_u16x2(m[2], v[u].z & 0x7FFF7FFFu);
                m[3] = max_u16x2(m[3], v[u].w & 0x7FFF7FFFu);
            }
        }
    } else if (c0 < K) {                        // the row's last, partial group of 8 columns
        for (int r = r0 + wave; r < r1; r += kWaves) {
            const uint16_t *p = X + (int64_t)r * ld + c0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < K) {
                    const uint32_t h = (uint32_t)(p[j] & 0x7FFF) << (16 * (j & 1));
                    m[j >> 1] = max_u16x2(m[j >> 1], h);
                }
        }
    }
    red[wave][lane] = uint4{m[0], m[1], m[2], m[3]};
    __syncthreads();
    if (wave == 0 && c0 < kp) {
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const uint4 o = red[w][lane];
            m[0] = max_u16x2(m[0], o.x);
            m[1] = max_u16x2(m[1], o.y);
            m[2] = max_u16x2(m[2], o.z);
            m[3] = max_u16x2(m[3], o.w);
        }
        *reinterpret_cast<uint4 *>(partial + (int64_t)blockIdx.y * kp + c0) = uint4{m[0], m[1], m[2], m[3]};
    }
}

// keys[c] = max over chunks of partial[chunk][c]. A workgroup takes 16
// groups of 8 channels; the 16 lanes of a group split the chunks between
// them (several loads in flight each) and meet in LDS. The optional fp16
// absmax output gets the same values (the sign bit is clear).
constexpr int kFoldGroups = 16, kFoldSlices = 16;

__global__ __launch_bounds__(kFoldGroups * kFoldSlices) void fold_kernel(const uint16_t *partial, int chunks,
                                                                         int64_t kp, int K, uint16_t *keys,
                                                                         uint16_t *absmax_out) {
    __shared__ uint4 red[kFoldSlices][kFoldGroups];
    const int g = threadIdx.x % kFoldGroups, sl = threadIdx.x / kFoldGroups;
    const int c0 = (blockIdx.x * kFoldGroups + g) * 8;
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    if (c0 < kp) {
#pragma unroll 4
        for (int ch = sl; ch < chunks; ch += kFoldSlices) {
            const uint4 v = *reinterpret_cast<const uint4 *>(partial + (int64_t)ch * kp + c0);
            m[0] = max_u16x2(m[0], v.x);
            m[1] = max_u16x2(m[1], v.y);
            m[2] = max_u16x2(m[2], v.z);
            m[3] = max_u16x2(m[3], v.w);
        }
    }
    red[sl][g] = uint4{m[0], m[1], m[2], m[3]};
    __syncthreads();
    if (sl != 0 || c0 >= kp)
        return;
#pragma unroll
    for (int t = 1; t < kFoldSlices; ++t) {
        const uint4 o = red[t][g];
        m[0] = max_u16x2(m[0], o.x);
        m[1] = max_u16x2(m[1], o.y);
        m[2] = max_u16x2(m[2], o.z);
        m[3] = max_u16x2(m[3], o.w);
    }
    *reinterpret_cast<uint4 *>(keys + c0) = uint4{m[0], m[1], m[2], m[3]};
    if (absmax_out)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c0 + j < K)
                absmax_out[c0 + j] = (uint16_t)(m[j >> 1] >> (16 * (j & 1)));
}

// Wave 0 finds, over bins visited from the highest down, the first bin at
// which the running count reaches `need`: returns that bin and the count of
// the bins above it. BPL bins per lane (64 * BPL bins in all).
template <int BPL>
__device__ void find_crossing(const uint32_t *hist, uint32_t need, int *bin_out, uint32_t *above_out) {
    const int lane = threadIdx.x & 63;
    const int nb = 64 * BPL;
    uint32_t h[BPL], s = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        h[j] = hist[nb - 1 - (lane * BPL + j)];
        s += h[j];
    }
    uint32_t incl = s;                         // inclusive scan over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    const uint64_t hit = __ballot(incl >= need);
    // the counts sum to at least `need`, so some lane crosses; the guard keeps
    // the bit scan defined even if that did not hold
    const int first = hit ? __builtin_ctzll(hit) : 63;
    if (lane == first) {
        uint32_t above = incl - s;
        int j = 0;
        while (j < BPL - 1 && above + h[j] < need) {
            above += h[j];
            ++j;
        }
        *bin_out = nb - 1 - (lane * BPL + j);
        *above_out = above;
    }
}

// Exclusive scan of one value per lane over the workgroup (1024 lanes).
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    if (lane == 63)
        wtot[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w)
        before += wtot[w];
    __syncthreads();                           // wtot is reused by the next scan
    return before + incl - v;
}

// Histogram copies: lane l adds into copy l % 4, so that lanes of one wave
// hitting the same bin are spread over four LDS banks (stride 260 words).
constexpr int kHistCopies = 4, kHistStride = 260;
constexpr int kKeysPerLane = kMaxK / kSelThreads;   // 32

__global__ __launch_bounds__(kSelThreads) void select_kernel(const uint16_t *keys_g, int64_t kp, int K, int n_out,
                                                             int32_t *out_idx, int32_t *perm) {
    __shared__ __align__(16) uint16_t key[kMaxK];
    __shared__ uint32_t hcopy[kHistCopies * kHistStride];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[kSelThreads / 64];
    __shared__ int sh_bin;
    __shared__ uint32_t sh_above;
    const int tid = threadIdx.x;
    {
        // 8 keys per 16-byte load (the keys past K up to kp are zero); all of
        // a lane's loads are issued before the first is stored
        constexpr int kLoads = kMaxK / 8 / kSelThreads;
        const int n8 = (int)(kp / 8);
        uint4 v[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int q = i * kSelThreads + tid;
            if (q < n8)
                v[i] = reinterpret_cast<const uint4 *>(keys_g)[q];
        }
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int q = i * kSelThreads + tid;
            if (q < n8)
                reinterpret_cast<uint4 *>(key)[q] = v[i];
        }
    }
    __syncthreads();

    // lane t owns channels [t P, t P + P), P a multiple of 8 (16-byte LDS
    // reads); its keys stay in registers, two per dword
    const int P = ((K + kSelThreads - 1) / kSelThreads + 7) / 8 * 8;
    const int b0 = min(tid * P, K), b1 = min(b0 + P, K);
    uint32_t kr[kKeysPerLane / 2];
#pragma unroll
    for (int q = 0; q < kKeysPerLane / 8; ++q) {
        const uint4 v = q * 8 < P && b0 + q * 8 < K ? reinterpret_cast<const uint4 *>(key + b0)[q]
                                                    : uint4{0u, 0u, 0u, 0u};
        kr[4 * q] = v.x;
        kr[4 * q + 1] = v.y;
        kr[4 * q + 2] = v.z;
        kr[4 * q + 3] = v.w;
    }
    auto key_at = [&](int i) { return (int)((kr[i >> 1] >> (16 * (i & 1))) & 0xFFFF); };
    uint32_t *my_hist = hcopy + (tid & (kHistCopies - 1)) * kHistStride;
    auto build_hist = [&](int level, int hb) {
        for (int t = tid; t < kHistCopies * kHistStride; t += kSelThreads)
            hcopy[t] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kKeysPerLane; ++i)
            if (i < b1 - b0) {
                const int k = key_at(i);
                if (level == 0)
                    atomicAdd(&my_hist[k >> 8], 1u);   // keys <= 0x7FFF: 128 high bins
                else if ((k >> 8) == hb)
                    atomicAdd(&my_hist[k & 255], 1u);
            }
        __syncthreads();
        if (tid < 256) {
            uint32_t h = 0;
#pragma unroll
            for (int c = 0; c < kHistCopies; ++c)
                h += hcopy[c * kHistStride + tid];
            hist[tid] = h;
        }
        __syncthreads();
    };

    // threshold T and the number of keys equal to T that are taken
    int T;
    uint32_t take_eq;
    if (n_out == 0) {
        T = 0x10000;                           // above every key: nothing selected
        take_eq = 0;
    } else if (n_out == K) {
        T = -1;                                // below every key: everything selected
        take_eq = 0;
    } else {
        build_hist(0, 0);
        if (tid < 64)
            find_crossing<2>(hist, (uint32_t)n_out, &sh_bin, &sh_above);
        __syncthreads();
        const int hb = sh_bin;
        const uint32_t above_hi = sh_above;
        __syncthreads();
        build_hist(1, hb);
        if (tid < 64)
            find_crossing<4>(hist, (uint32_t)n_out - above_hi, &sh_bin, &sh_above);
        __syncthreads();
        T = (hb << 8) | sh_bin;
        take_eq = (uint32_t)n_out - above_hi - sh_above;
    }

    // channels in index order
    const int nk = b1 - b0;
    uint32_t eq = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
        eq += i < nk && key_at(i) == T;
    uint32_t eq_seen = block_exclusive_scan(eq, wtot);
    uint32_t nsel = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
        if (i < nk) {
            const int k = key_at(i);
            nsel += k > T || (k == T && eq_seen++ < take_eq);
        }
    uint32_t pos = block_exclusive_scan(nsel, wtot);   // selected channels before b0
    eq_seen -= eq;                                     // replay the same decisions
    const int head = K - n_out;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        if (i >= nk)
            break;
        const int c = b0 + i, k = key_at(i);
        if (k > T || (k == T && eq_seen++ < take_eq)) {
            if (out_idx)
                out_idx[pos] = c;
            perm[head + pos] = c;
            ++pos;
        } else {
            perm[c - pos] = c;
        }
    }
}

}  // namespace select_impl

SelectPlan plan_select(int32_t rows, int32_t K) {
    using namespace select_impl;
    SelectPlan p;
    p.stripes = (K + kStripe - 1) / kStripe;
    p.kp = (K + 7) / 8 * 8;
    if (rows <= 0) {
        p.chunks = 0;
        p.rows_per_chunk = 0;
    } else {
        const long want = std::max<long>(1, kTargetGroups / p.stripes);   // one wave of workgroups
        const long most = std::max<long>(1, (rows + kMinRowsPerChunk - 1) / kMinRowsPerChunk);
        const long chunks = std::min(want, most);
        p.rows_per_chunk = (int)((rows + chunks - 1) / chunks);
        p.chunks = (rows + p.rows_per_chunk - 1) / p.rows_per_chunk;
    }
    const size_t part = (size_t)p.chunks * p.kp * 2;
    p.keys_offset = (part + 255) / 256 * 256;
    p.workspace_bytes = p.keys_offset + (size_t)p.kp * 2;
    return p;
}

int select_max_k() { return select_impl::kMaxK; }

hipError_t launch_select(const SelectArgs &a, hipStream_t stream) {
    using namespace select_impl;
    const SelectPlan p = plan_select(a.rows, a.K);
    uint16_t *partial = static_cast<uint16_t *>(a.workspace);
    uint16_t *keys = reinterpret_cast<uint16_t *>(static_cast<char *>(a.workspace) + p.keys_offset);
    if (p.chunks > 0)
        hipLaunchKernelGGL(colmax_kernel, dim3(p.stripes, p.chunks), dim3(kWaves * 64), 0, stream,
                           static_cast<const uint16_t *>(a.X), a.ld, a.rows, a.K, p.rows_per_chunk, p.kp, partial);
    const int fold_groups = (int)((p.kp / 8 + kFoldGroups - 1) / kFoldGroups);
    hipLaunchKernelGGL(fold_kernel, dim3(fold_groups), dim3(kFoldGroups * kFoldSlices), 0, stream, partial, p.chunks,
                       p.kp, a.K, keys, static_cast<uint16_t *>(a.absmax));
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(kSelThreads), 0, stream, keys, p.kp, a.K, a.n_out,
                       a.outlier_idx, a.perm);
    return hipGetLastError();
}

}  // namespace w4a4
