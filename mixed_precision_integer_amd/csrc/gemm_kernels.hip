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
// CDNA4 design
// * CDNA4 has no INT4 matrix instruction, so packed nibbles are widened
//   exactly to int8 in registers: for a packed dword p,
//     hi = p & 0xF0F0F0F0         -> four int8 lanes holding 16 * q_odd
//     lo = (p << 4) & 0xF0F0F0F0  -> four int8 lanes holding 16 * q_even
//   (the sign comes for free from the two's complement nibble). Both
//   operands carry the factor 16, so the int32 accumulator holds 256 * acc,
//   exact while K_n * 64 * 256 < 2^31; the epilogue folds 2^-8 into the fp32
//   scale and the accumulator export shifts right by 8.
// * The nibble order inside an MFMA operand need not follow the channel
//   order: a dot product is invariant under one permutation of K applied to
//   both operands, and A and B are unpacked identically, so the widened
//   dwords go to v_mfma_i32_32x32x32_i8 as they come.
// * A K-tile is 64 bytes of every row: 128 INT4 channels or 64 INT8 tail
//   channels. The tail tiles run first as one scale group, then the INT4
//   tiles (a group per `group` channels, or one group for per-row scales).
//   The first MFMA of a group reads a zero C operand, so no accumulator is
//   ever cleared; at the end of a group the int32 sums are converted and
//   added into fp32 accumulators.
// * Tiles reach LDS through direct global->LDS DMA (global_load_lds_dwordx4,
//   issued as inline asm with a uniform base and 32-bit lane offsets): no VGPR
//   staging and no ds_write. A 4-stage LDS ring with prefetch
//   distance 2 needs one barrier per tile: the stage written at tile t was
//   last read at tile t-2, which every wave has finished once it has passed
//   the barrier of tile t-1. Every wave waits for its own DMA with an explicit
//   vmcnt before that barrier.
// * LDS rows are 64 bytes = four 16-byte chunks; chunk c of row r is stored
//   at slot (c ^ (r >> 1) ^ (r >> 2)) & 3. Any 8 consecutive rows then land on
//   8 distinct 16-byte slots modulo 128 bytes and any 16 on 16 distinct slots
//   modulo 256 bytes, so a ds_read_b128 of 32 rows is conflict-free whether
//   the banks serve 8 or 16 lanes per pass.
// * The fp32 scales of a tile's group ride along with every tile (DMA
//   dwords), so each tile costs the same number of DMA instructions and the
//   vmcnt bookkeeping is a constant.
// * Workgroups are mapped so that each XCD (own L2) works on a contiguous
//   range of tiles, walked in bands of 8 tile rows.
#include <algorithm>

#include "w4a4.h"
#include "gemm_common.h"

namespace w4a4 {
namespace gemm_impl {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    // LDS ring depth; tiles in flight ahead of the one being multiplied
    static constexpr int STAGES = STAGES_, PREFETCH = STAGES_ - 2;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int DA = BM * 4 / kThreads, DB = BN * 4 / kThreads;
    static constexpr int DS = (BM + BN + kThreads - 1) / kThreads;  // scale DMAs per lane
    static constexpr int A_BYTES = BM * kTileBytes, B_BYTES = BN * kTileBytes;
    static constexpr int S_BYTES = DS * kThreads * 4;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(DA >= 1 && DB >= 1 && BM * 4 % kThreads == 0 && BN * 4 % kThreads == 0, "loader");
    static_assert(PREFETCH >= 1 && PREFETCH <= 6, "ring depth");
};

// MFMAs of one K-tile held in LDS stage `st`. FRESH: the tile opens a scale
// group (its first MFMAs take C = 0). TAIL: an INT8 tail tile (no widening).
template <class C, bool FRESH, bool TAIL>
__device__ __forceinline__ void mma_tile(v16i (&acc)[C::FM][C::FN], const unsigned char *st, int wm,
                                         int wn, int li, int lh) {
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const unsigned char *sA = st, *sB = st + C::A_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + lh;
        uint4 pa[C::FM], pb[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            pa[fm] = *reinterpret_cast<const uint4 *>(sA + swz(wm * C::WTM + fm * 32 + li, c));
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
            pb[fn] = *reinterpret_cast<const uint4 *>(sB + swz(wn * C::WTN + fn * 32 + li, c));
        const bool z = FRESH && s == 0;
        if constexpr (TAIL) {
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) {
                    const v4i x = {(int)pa[fm].x, (int)pa[fm].y, (int)pa[fm].z, (int)pa[fm].w};
                    const v4i w = {(int)pb[fn].x, (int)pb[fn].y, (int)pb[fn].z, (int)pb[fn].w};
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x, w, z ? zero : acc[fm][fn], 0, 0, 0);
                }
        } else {
            v4i wb0[C::FN], wb1[C::FN];
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
                wb0[fn] = v4i{(int)nib_lo(pb[fn].x), (int)nib_hi(pb[fn].x), (int)nib_lo(pb[fn].y),
                              (int)nib_hi(pb[fn].y)};
                wb1[fn] = v4i{(int)nib_lo(pb[fn].z), (int)nib_hi(pb[fn].z), (int)nib_lo(pb[fn].w),
                              (int)nib_hi(pb[fn].w)};
            }
            // first halves of every block, then second halves: consecutive MFMAs
            // never chain on one accumulator
            v4i xa1[C::FM];
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
                const v4i xa0 = {(int)nib_lo(pa[fm].x), (int)nib_hi(pa[fm].x), (int)nib_lo(pa[fm].y),
                                 (int)nib_hi(pa[fm].y)};
                xa1[fm] = v4i{(int)nib_lo(pa[fm].z), (int)nib_hi(pa[fm].z), (int)nib_lo(pa[fm].w),
                              (int)nib_hi(pa[fm].w)};
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa0, wb0[fn], z ? zero : acc[fm][fn], 0, 0, 0);
            }
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa1[fm], wb1[fn], acc[fm][fn], 0, 0, 0);
        }
    }
}

// End of a scale group: y += float(acc) * (sa[m] * sw[n]) (the INT4 sums also
// * 2^-8), with the group's scales read from the LDS stage of its last tile:
// floats [0, BM) are the row scales, [BM, BM + BN) the column scales.
template <class C, bool TAIL>
__device__ __forceinline__ void dequant_group(const v16i (&acc)[C::FM][C::FN],
                                              float (&yacc)[C::FM][C::FN][16],
                                              const unsigned char *st, int wm, int wn, int li,
                                              int lh) {
    const float *sS = reinterpret_cast<const float *>(st + C::A_BYTES + C::B_BYTES);
    constexpr float unit = TAIL ? 1.0f : (1.0f / 256.0f);
    float cs[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
        cs[fn] = sS[C::BM + wn * C::WTN + fn * 32 + li] * unit;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        float rs[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(sS + wm * C::WTM + fm * 32 + q * 8 + lh * 4);
            rs[q * 4 + 0] = v.x;
            rs[q * 4 + 1] = v.y;
            rs[q * 4 + 2] = v.z;
            rs[q * 4 + 3] = v.w;
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                yacc[fm][fn][r] = __builtin_fmaf((float)acc[fm][fn][r], rs[r] * cs[fn], yacc[fm][fn][r]);
    }
}

// Accumulator export (test path): add the exact integer sums of a group (or,
// under a K split, of the part of the group this split covers).
template <class C, bool TAIL>
__device__ __forceinline__ void export_group(const v16i (&acc)[C::FM][C::FN], const GemmArgs &a,
                                             int gidx, int row0, int col0, int wm, int wn, int li,
                                             int lh) {
    int32_t *dst = TAIL ? a.acc8_out : a.acc4_out + (int64_t)gidx * a.M * a.N;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const int n = col0 + wn * C::WTN + fn * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = row0 + wm * C::WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                const int v = acc[fm][fn][r];
                if (m < a.M && n < a.N)
                    export_add(dst + (int64_t)m * a.N + n, TAIL ? v : (v >> 8));
            }
        }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    compiler_fence();
}

template <class C, bool EXPORT, bool SPLIT>
__device__ __forceinline__ void gemm_body(const GemmArgs &a) {
    constexpr int BM = C::BM, BN = C::BN, FM = C::FM, FN = C::FN;
    constexpr int STAGES = C::STAGES, PREFETCH = C::PREFETCH;
    constexpr int STAGE = C::A_BYTES + C::B_BYTES + C::S_BYTES;
    constexpr int D = C::DA + C::DB + C::DS;                   // DMA instructions per tile per lane

    __shared__ __align__(16) unsigned char lds[STAGES * STAGE];
    __shared__ int last_split;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int li = lane & 31, lh = lane >> 5;

    // ---- output tile and K split of this workgroup ------------------------------
    const int S = SPLIT ? a.splits : 1;
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int ks = blockIdx.x % S;
    const int tile = blockIdx.x / S;
    int tm, tn;
    tile_coords(tile, tiles_m, tiles_n, S == 1, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    const int T8 = (int)(a.pitch8 / kTileBytes);
    const int T4 = (int)(a.pitch4 / kTileBytes);
    const int T = T8 + T4;
    // INT4 tiles per scale group (per-row scales: all of them). With no INT4
    // channels (every channel an outlier) there are no INT4 groups.
    const int tiles_per_group = a.group > 0 ? a.group / 128 : max(T4, 1);
    // K-tiles [t_begin, t_end) of this split; split boundaries may cut a scale
    // group, whose two parts are then dequantized with the same scales.
    const int t_begin = (int)((int64_t)ks * T / S), t_end = (int)((int64_t)(ks + 1) * T / S);

    // ---- DMA sources of this lane ----------------------------------------------
    // Slot q = j * 256 + tid of a tile holds row r = q / 4, chunk (q % 4) ^ f(r).
    // Per-lane byte offsets are fixed for the whole K loop; only the uniform
    // base (operand pointer + 64 * tile) moves.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t a4o[C::DA], a8o[C::DA], b4o[C::DB], b8o[C::DB];
#pragma unroll
    for (int j = 0; j < C::DA; ++j) {
        const int q = j * kThreads + tid, r = q >> 2;
        const uint32_t row = min(row0 + r, a.M - 1);
        const uint32_t off = dma_chunk_offset(q);
        a4o[j] = row * (uint32_t)a.pitch4 + off;
        a8o[j] = row * (uint32_t)a.pitch8 + off;
    }
#pragma unroll
    for (int j = 0; j < C::DB; ++j) {
        const int q = j * kThreads + tid, r = q >> 2;
        const uint32_t row = min(col0 + r, a.N - 1);
        const uint32_t off = dma_chunk_offset(q);
        b4o[j] = row * (uint32_t)a.pitch4 + off;
        b8o[j] = row * (uint32_t)a.pitch8 + off;
    }
    // scale slots: rows of A first, then columns of B
    bool s_is_a[C::DS];
    uint32_t s_row[C::DS];
#pragma unroll
    for (int j = 0; j < C::DS; ++j) {
        const int e = min(j * kThreads + tid, BM + BN - 1);
        s_is_a[j] = e < BM;
        s_row[j] = e < BM ? min(row0 + e, a.M - 1) : min(col0 + e - BM, a.N - 1);
    }

    auto issue = [&](int tt) {
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE;
        const uint32_t sa = st + wave_u * 1024, sb = st + C::A_BYTES + wave_u * 1024;
        const uint32_t ss = st + C::A_BYTES + C::B_BYTES + wave_u * 256;
        if (tt < T8) {
            const uint8_t *A = reinterpret_cast<const uint8_t *>(a.a8) + tt * kTileBytes;
            const uint8_t *B = reinterpret_cast<const uint8_t *>(a.w8) + tt * kTileBytes;
#pragma unroll
            for (int j = 0; j < C::DA; ++j)
                dma16(A, a8o[j], sa + j * 4096);
#pragma unroll
            for (int j = 0; j < C::DB; ++j)
                dma16(B, b8o[j], sb + j * 4096);
#pragma unroll
            for (int j = 0; j < C::DS; ++j)
                dma4((s_is_a[j] ? a.sa8 : a.sw8) + s_row[j], ss + j * 1024);
        } else {
            const int t4 = tt - T8;
            const uint8_t *A = a.a4 + t4 * kTileBytes;
            const uint8_t *B = a.w4 + t4 * kTileBytes;
#pragma unroll
            for (int j = 0; j < C::DA; ++j)
                dma16(A, a4o[j], sa + j * 4096);
#pragma unroll
            for (int j = 0; j < C::DB; ++j)
                dma16(B, b4o[j], sb + j * 4096);
            const int g = t4 / tiles_per_group;
#pragma unroll
            for (int j = 0; j < C::DS; ++j)
                dma4((s_is_a[j] ? a.sa4 : a.sw4) + s_row[j] * (uint32_t)a.G + g, ss + j * 1024);
        }
    };

    // Wait for tile tt (after issuing tile tt + PREFETCH if it is in this
    // split) and make it visible to the whole workgroup. Tiles after tt that
    // are already in flight stay in flight.
    auto begin_tile = [&](int tt) -> const unsigned char * {
        compiler_fence();
        if (tt + PREFETCH < t_end) {
            issue(tt + PREFETCH);
            if constexpr (EXPORT)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // accumulator stores share vmcnt
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(PREFETCH * D));
        } else if constexpr (EXPORT) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        } else {
            wait_tiles<D>(t_end - 1 - tt);
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

    // ---- main loop: the tail group, then the INT4 groups ------------------------------
#pragma unroll
    for (int p = 0; p < PREFETCH; ++p)
        if (t_begin + p < t_end)
            issue(t_begin + p);

    int tt = t_begin;
    if (tt < T8) {
        const int run_end = min(T8, t_end);
        const unsigned char *st = begin_tile(tt++);
        mma_tile<C, true, true>(acc, st, wm, wn, li, lh);
        while (tt < run_end) {
            st = begin_tile(tt++);
            mma_tile<C, false, true>(acc, st, wm, wn, li, lh);
        }
        if constexpr (EXPORT)
            export_group<C, true>(acc, a, 0, row0, col0, wm, wn, li, lh);
        dequant_group<C, true>(acc, yacc, st, wm, wn, li, lh);
    }
    while (tt < t_end) {
        const int g = (tt - T8) / tiles_per_group;
        const int run_end = min(T8 + (g + 1) * tiles_per_group, t_end);
        const unsigned char *st = begin_tile(tt++);
        mma_tile<C, true, false>(acc, st, wm, wn, li, lh);
        while (tt < run_end) {
            st = begin_tile(tt++);
            mma_tile<C, false, false>(acc, st, wm, wn, li, lh);
        }
        if constexpr (EXPORT)
            export_group<C, false>(acc, a, g, row0, col0, wm, wn, li, lh);
        dequant_group<C, false>(acc, yacc, st, wm, wn, li, lh);
    }

    {
        if constexpr (!SPLIT) {
            // ---- epilogue: fp16 store --------------------------------------------------
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int n = col0 + wn * C::WTN + fn * 32 + li;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = row0 + wm * C::WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                        if (m < a.M && n < a.N)
                            a.y[(int64_t)m * a.ldy + n] = (_Float16)yacc[fm][fn][r];
                    }
                }
        } else {
            // ---- split-K epilogue ------------------------------------------------------
            // Every split stores its fp32 partial tile; the last split of the tile
            // to arrive (device-wide counter) adds the S partials in split order,
            // so the result does not depend on which one that is, writes fp16 and
            // returns the counter to zero for the next call.
            // The partials and the counter are touched only by agent-scope
            // relaxed atomics, which are coherent across the XCDs' L2s without
            // a whole-cache write-back or invalidate; the partial stores are
            // complete (vmcnt 0) before the counter is incremented, and the
            // reads are issued only after the increment has returned.
            float *part = a.part + (int64_t)ks * a.M * a.N;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int n = col0 + wn * C::WTN + fn * 32 + li;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = row0 + wm * C::WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                        if (m < a.M && n < a.N)
                            __hip_atomic_store(part + (int64_t)m * a.N + n, yacc[fm][fn][r],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            compiler_fence();
            __syncthreads();
            if (tid == 0) {
                const uint32_t prev = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                const int is_last = prev == (uint32_t)(S - 1);
                if (is_last)
                    __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_split = is_last;
            }
            __syncthreads();
            if (last_split) {
                // Partials of up to kSB splits for all of this lane's elements are
                // loaded as one batch (every load in bounds: rows past M and
                // splits past S are clamped and their values discarded), so the
                // batch costs one memory latency.
                constexpr int kSB = 4;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const int n = col0 + wn * C::WTN + fn * 32 + li;
                        const int ncl = min(n, a.N - 1);
                        float sum[16];
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sum[r] = 0.0f;
                        for (int s0 = 0; s0 < S; s0 += kSB) {
                            float v[kSB][16];
#pragma unroll
                            for (int j = 0; j < kSB; ++j) {
                                const float *src = a.part + (int64_t)min(s0 + j, S - 1) * a.M * a.N;
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int m = row0 + wm * C::WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                                    v[j][r] = __hip_atomic_load(src + (int64_t)min(m, a.M - 1) * a.N + ncl,
                                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                }
                            }
#pragma unroll
                            for (int j = 0; j < kSB; ++j)
                                if (s0 + j < S)
#pragma unroll
                                    for (int r = 0; r < 16; ++r)
                                        sum[r] += v[j][r];
                        }
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = row0 + wm * C::WTM + fm * 32 + (r / 4) * 8 + lh * 4 + (r % 4);
                            if (m < a.M && n < a.N)
                                a.y[(int64_t)m * a.ldy + n] = (_Float16)sum[r];
                        }
                    }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool EXPORT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
    gemm_body<Cfg<BM, BN, WAVES_M, WAVES_N, STAGES>, EXPORT, SPLIT>(a);
}

template <class C, bool EXPORT>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
    const dim3 grid(tiles * a.splits);
    if (a.splits > 1)
        hipLaunchKernelGGL((gemm_kernel<C::BM, C::BN, C::WAVES_M, C::WAVES_N, C::STAGES, EXPORT, true>), grid,
                           dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<C::BM, C::BN, C::WAVES_M, C::WAVES_N, C::STAGES, EXPORT, false>), grid,
                           dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

using CfgMid = Cfg<128, 128, 2, 2, 4>;     // waves of 64 x 64, two workgroups per CU
using CfgSmall = Cfg<64, 64, 2, 2, 4>;     // waves of 32 x 32, four workgroups per CU

}  // namespace gemm_impl

using namespace gemm_impl;

namespace {

constexpr int kDeviceCUs = 256;            // MI355X; the split choice is tuned for it
constexpr int kMaxSplitTiles = kDeviceCUs * 2;   // a shape splits K only below this
constexpr size_t kSplitCounterBytes = (kMaxSplitTiles * sizeof(uint32_t) + 255) / 256 * 256;

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

size_t gemm_counter_bytes() { return kSplitCounterBytes; }

// Name of the production kernel of a plan as the kernel trace prints it
// (template arguments included where they are fixed by the shape).
const char *gemm_kernel_name(const GemmPlan &p) {
    switch (p.cfg) {
    case 0: return p.splits > 1 ? "gemm_kernel<64, 64, 2, 2, 4, false, true>" : "gemm_kernel<64, 64, 2, 2, 4, false, false>";
    case 1: return p.splits > 1 ? "gemm_kernel<128, 128, 2, 2, 4, false, true>" : "gemm_kernel<128, 128, 2, 2, 4, false, false>";
    case 2: return "gemm_big_kernel";
    case 3: return "gemm_group_kernel<false>";
    case 4: return decode_kernel_name(p.rows);
    default: return "unknown";
    }
}

// Tile shape and K split for a shape. A pure function of the shape, so the
// workspace query and the launch always agree, and the accumulator export
// runs the same kernel as the product.
GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group) {
    GemmPlan p{};
    if (gemm_decode_fits(M, N, K_n, n_out, group)) {
        p.cfg = 4;
        p.tiles = ceil_div(N, 32);
        p.splits = 1;
        p.mb = ceil_div(M, 32);
        p.rows = M;
        return p;
    }
    if (gemm_big_fits(M, N, K_n, n_out, w4a4_num_groups(K_n, group))) {
        p.cfg = 2;
        p.tiles = ((M + 255) / 256) * ((N + 255) / 256);
        p.splits = 1;
        return p;
    }
    const bool small = M <= 64;
    const int bm = small ? CfgSmall::BM : CfgMid::BM, bn = small ? CfgSmall::BN : CfgMid::BN;
    const int per_cu = small ? 4 : 2;                          // resident workgroups per CU (LDS)
    p.cfg = small ? 0 : 1;
    p.tiles = ceil_div(M, bm) * ceil_div(N, bn);
    const int T = (int)(w4a4_pitch4_bytes(K_n) / 64 + w4a4_pitch8_bytes(n_out) / 64);
    int S = 1;
    const int slots = kDeviceCUs * per_cu;
    if (p.tiles > 0 && p.tiles * 2 <= slots && p.tiles <= kMaxSplitTiles) {
        // about half the resident slots: measured on the 8192 x 8192 decode
        // shapes, more splits cost more in partial-sum traffic and arrival
        // latency than they gain in memory parallelism. At least two K-tiles
        // per split, and the fp32 partial traffic (S * M * N * 8 bytes) at most
        // the packed weights' size (N * K_n / 2).
        S = ceil_div(slots / 2, p.tiles);
        S = std::min(S, std::max(1, T / 2));
        S = std::min(S, std::max(1, (int)(K_n / 8 / std::max(M, 1))));
        S = std::min(S, 32);
        S = std::max(S, 1);
    }
    p.splits = S;
    if (S == 1 && gemm_group_fits(M, N, K_n, n_out, group)) {
        p.cfg = 3;
        p.tiles = ceil_div(M, 128) * ceil_div(N, 128);
        return p;
    }
    if (S > 1) {
        // The counters sit at a fixed place, first in the workspace, sized for
        // the most tiles that are ever split: partial sums of one shape then
        // never land on the counters of another, and a zeroed workspace stays
        // valid for calls of any shape.
        p.part_offset = kSplitCounterBytes;
        p.part_bytes = (size_t)S * M * N * sizeof(float);
        p.workspace_bytes = p.part_offset + p.part_bytes;
    }
    return p;
}

namespace {

__global__ void zero_i32_kernel(int32_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride)
        p[j] = 0;
}

hipError_t zero_i32(int32_t *p, int64_t n, hipStream_t stream) {
    if (!p || n <= 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace

hipError_t clear_gemm_counters(void *workspace, hipStream_t stream) {
    return zero_i32(static_cast<int32_t *>(workspace), (int64_t)(kSplitCounterBytes / sizeof(int32_t)), stream);
}

hipError_t launch_gemm(const GemmArgs &a_in, bool export_acc, void *workspace, hipStream_t stream) {
    if (a_in.M == 0 || a_in.N == 0)
        return hipSuccess;
    GemmArgs a = a_in;
    const GemmPlan p = plan_gemm(a.M, a.N, a.K_n, a.n_out, a.group);
    a.splits = p.splits;
    if (p.splits > 1) {
        a.ctr = static_cast<uint32_t *>(workspace);
        a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + p.part_offset);
    }
    if (export_acc) {
        // the export adds partial sums: both arrays start at zero
        hipError_t e = zero_i32(a.acc4_out, (int64_t)a.G * a.M * a.N, stream);
        if (e == hipSuccess && a.n_out > 0)
            e = zero_i32(a.acc8_out, (int64_t)a.M * a.N, stream);
        if (e != hipSuccess)
            return e;
    } else {
        a.acc4_out = nullptr;
        a.acc8_out = nullptr;
    }
    if (p.cfg == 2)
        return launch_gemm_big(a, export_acc, stream);
    if (p.cfg == 3)
        return launch_gemm_group(a, export_acc, stream);
    if (p.cfg == 4)
        return launch_gemm_decode(a, export_acc, stream);
    if (p.cfg == 0)
        return export_acc ? launch_cfg<CfgSmall, true>(a, stream) : launch_cfg<CfgSmall, false>(a, stream);
    return export_acc ? launch_cfg<CfgMid, true>(a, stream) : launch_cfg<CfgMid, false>(a, stream);
}

}  // namespace w4a4
