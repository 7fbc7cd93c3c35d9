// Large-shape GEMM for per-row scales: 256 x 256 output tile per workgroup,
// four waves of 128 x 128, int32 accumulators in AGPRs (this translation
// unit is built without the VGPR accumulator form).
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part plus an
// 8-bit outlier part over reordered channels; Key points item 5: symmetric
// scales factor out of the integer sums) and the QUIK abstract (hybrid
// 4-bit layer with higher-precision outliers). With one scale per row and
// one per column for the INT4 head (and for the INT8 tail), the whole K loop
// accumulates exact integers and dequantization happens once per output.
//
// CDNA4 design (see gemm_kernels.hip for the widening and the LDS layout,
// which are shared)
// * A wave owns 4 x 4 blocks of 32 x 32, so each widened operand fragment
//   feeds four MFMAs: 3 VALU ops per v_mfma_i32_32x32x32_i8 for the nibble
//   widening, below what a lone wave can issue beside its MFMAs. The 256
//   accumulator registers are AGPRs, written by the MFMAs directly; one wave
//   per SIMD.
// * K-tiles of 64 bytes per row (128 INT4 channels) reach a 4-stage LDS ring
//   (32 KB per stage) by direct global->LDS DMA, prefetch distance 2, one
//   barrier per tile.
// * The INT8 outlier tail (at most four K-tiles) is loaded last and kept in
//   the ring whole; the epilogue multiplies it block by block into a 16-
//   register accumulator, so the tail needs no second 256-register set.
// * y = fp16(acc8 * (sa8 * sw8) + acc4 * (sa4 * sw4 / 256)), rows and columns
//   guarded at the ragged edges.
#include <algorithm>

#include "w4a4.h"
#include "gemm_common.h"

namespace w4a4 {
namespace gemm_big_impl {

using namespace gemm_impl;

constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128, FM = 4, FN = 4;
constexpr int STAGES = 4, PREFETCH = 3;         // K-tiles in flight beyond the one being read
constexpr int A_BYTES = BM * kTileBytes, B_BYTES = BN * kTileBytes;
constexpr int STAGE = A_BYTES + B_BYTES;                 // 32 KB
constexpr int DA = BM * 4 / kThreads, DB = BN * 4 / kThreads;
constexpr int D = DA + DB;                               // DMA instructions per tile per lane
constexpr int MAX_TAIL_TILES = STAGES;
constexpr int SCALE_BYTES = 4 * BM * 4;                // sa4, sa8, sw4, sw8 of the tile (BM == BN)
// Per-wave fp16 staging of the interior epilogue: 32 rows x 64 columns, rows
// padded by 16 bytes so the eight-byte writes of a column of lanes spread
// over the banks.
constexpr int STG_PITCH = 64 * 2 + 16;
constexpr int STG_BYTES = 32 * STG_PITCH;
constexpr int LDS_BYTES = STAGES * STAGE + SCALE_BYTES + 4 * STG_BYTES;

// Raw packed fragments of one sub-step (64 channels) of a K-tile: lane
// (li, lh) reads 16 bytes of row li of each 32-row block, chunk 2 s + lh.
struct Frag {
    uint4 a[FM], b[FN];
};
// The same, widened to int8 lanes holding 16 * q: x0/w0 feed the first
// 32-channel k-step, x1/w1 the second.
struct Wide {
    v4i x0[FM], x1[FM], w0[FN], w1[FN];
};

// Fragment i of a sub-step: i < 4 is row block i of the activation tile,
// i >= 4 column block i - 4 of the weight tile (16 bytes per lane, chunk
// 2 s + lh of row li of the block).
__device__ __forceinline__ uint4 read_one(const unsigned char *st, int i, int s, int wm, int wn, int li, int lh) {
    const int c = 2 * s + lh;
    return i < 4 ? *reinterpret_cast<const uint4 *>(st + swz(wm * WTM + i * 32 + li, c))
                 : *reinterpret_cast<const uint4 *>(st + A_BYTES + swz(wn * WTN + (i - 4) * 32 + li, c));
}

__device__ __forceinline__ void read_frag(Frag &f, const unsigned char *st, int s, int wm, int wn, int li, int lh) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 v = read_one(st, i, s, wm, wn, li, lh);
        if (i < 4)
            f.a[i] = v;
        else
            f.b[i - 4] = v;
    }
}

// Widen fragment i (3 VALU ops per packed dword pair of int8 lanes).
__device__ __forceinline__ void widen_one(Wide &w, const Frag &f, int i) {
    if (i < 4) {
        const uint4 p = f.a[i];
        w.x0[i] = v4i{(int)nib_lo(p.x), (int)nib_hi(p.x), (int)nib_lo(p.y), (int)nib_hi(p.y)};
        w.x1[i] = v4i{(int)nib_lo(p.z), (int)nib_hi(p.z), (int)nib_lo(p.w), (int)nib_hi(p.w)};
    } else {
        const uint4 p = f.b[i - 4];
        w.w0[i - 4] = v4i{(int)nib_lo(p.x), (int)nib_hi(p.x), (int)nib_lo(p.y), (int)nib_hi(p.y)};
        w.w1[i - 4] = v4i{(int)nib_lo(p.z), (int)nib_hi(p.z), (int)nib_lo(p.w), (int)nib_hi(p.w)};
    }
}

__device__ __forceinline__ void widen(Wide &w, const Frag &f) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        widen_one(w, f, i);
}

// MFMAs i of a sub-step's 8 groups of four: the first k-step (x0, w0) of
// row block i for i < 4, the second (x1, w1) of row block i - 4 otherwise;
// each over the four column blocks. The weight fragment is the MFMA's first
// operand, so block (fm, fn) accumulates the transposed product: lane (li, lh)
// holds output row li of the block and the 16 columns 8 * (r / 4) + 4 * lh +
// r % 4, four consecutive ones per r / 4. Consecutive MFMAs never chain on
// one accumulator.
__device__ __forceinline__ void mma_four(v16i (&acc)[FM][FN], const Wide &w, int i) {
    const int fm = i & 3;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = i < 4 ? __builtin_amdgcn_mfma_i32_32x32x32_i8(w.w0[fn], w.x0[fm], acc[fm][fn], 0, 0, 0)
                            : __builtin_amdgcn_mfma_i32_32x32x32_i8(w.w1[fn], w.x1[fm], acc[fm][fn], 0, 0, 0);
}

// Order inside one chunk: each MFMA followed by three VALU ops, the LDS
// reads after the first MFMA.
template <int READS>
__device__ __forceinline__ void chunk_order() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    if constexpr (READS > 0)
        __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
}

// y = acc4 * s4 + acc8 * s8 with the roundings spelled out (one product,
// then one fused multiply-add, rounded to fp32 before the fp16 conversion),
// so that both epilogues, and the accumulator export's launch, give the same
// bits whatever the compiler would contract (left alone, it fuses the last
// FMA of one epilogue with the fp16 conversion into v_fma_mixlo_f16, one
// rounding instead of two).
__device__ __forceinline__ float y_value(int acc4, int acc8, float s4, float s8) {
#pragma clang fp contract(off)
    const float p4 = (float)acc4 * s4;
    float y = __builtin_fmaf((float)acc8, s8, p4);
    asm volatile("" : "+v"(y));
    return y;
}

// fp16 pair, round to nearest even, packed low | high << 16
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    const _Float16 l = (_Float16)lo, h = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Epilogue of edge tiles (and, in the accumulator export, of every tile: the
// exact sums are stored, then Y as in the production epilogue), block by block
// (column block outer, so the weight side of the tail is read once per
// column): the INT4 sums of the block are copied out (and converted to the
// fp32 partial acc4 * (sa4 * sw4 / 256), or exported), the INT8 tail product
// is accumulated in place on top of them, always over MAX_TAIL_TILES tiles
// with the weight operand zeroed past the tail, and recovered as the
// difference; y = fp16(partial + acc8 * (sa8 * sw8)). Stores are guarded
// element by element at the ragged edges.
template <bool EXPORT>
__device__ __forceinline__ void epilogue(const GemmArgs &a, v16i (&acc)[FM][FN], const unsigned char *lds,
                                         const float *sS, int T4, int T8, int row0, int col0, int wm, int wn,
                                         int li, int lh) {
    const bool vec_store = ((reinterpret_cast<uintptr_t>(a.y) | (uintptr_t)(a.ldy * 2)) & 7) == 0;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int nl = wn * WTN + fn * 32 + lh * 4;        // tile-local first column of the lane
        v4i pb8[MAX_TAIL_TILES][2];
#pragma unroll
        for (int j = 0; j < MAX_TAIL_TILES; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint4 p = *reinterpret_cast<const uint4 *>(lds + ((T4 + j) % STAGES) * STAGE + A_BYTES +
                                                                swz(wn * WTN + fn * 32 + li, 2 * s + lh));
                pb8[j][s] = j < T8 ? v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w} : v4i{0, 0, 0, 0};
            }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int ml = wm * WTM + fm * 32 + li;
            const int m = row0 + ml;
            int a4[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                a4[r] = acc[fm][fn][r];
#pragma unroll
            for (int j = 0; j < MAX_TAIL_TILES; ++j)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint4 p = *reinterpret_cast<const uint4 *>(lds + ((T4 + j) % STAGES) * STAGE + swz(ml, 2 * s + lh));
                    const v4i x = {(int)p.x, (int)p.y, (int)p.z, (int)p.w};
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(pb8[j][s], x, acc[fm][fn], 0, 0, 0);
                }
            if constexpr (EXPORT) {
                // accumulator export (test path): this workgroup owns the sums
                if (m < a.M) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int n = col0 + nl + (r / 4) * 8 + (r % 4);
                        if (n < a.N) {
                            const int64_t e = (int64_t)m * a.N + n;
                            a.acc4_out[e] = a4[r] >> 8;
                            if (a.acc8_out)
                                a.acc8_out[e] = acc[fm][fn][r] - a4[r];
                        }
                    }
                }
            }
            {
                const float rs4 = sS[ml] * (1.0f / 256.0f);
                const float rs8 = T8 > 0 ? sS[BM + ml] : 0.0f;   // tail scales are not loaded when T8 == 0
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(sS + 2 * BM + nl + q * 8);
                    const float4 c8v = *reinterpret_cast<const float4 *>(sS + 3 * BM + nl + q * 8);
                    const float4 c8 = T8 > 0 ? c8v : float4{0.0f, 0.0f, 0.0f, 0.0f};
                    const float cs4[4] = {c4.x, c4.y, c4.z, c4.w}, cs8[4] = {c8.x, c8.y, c8.z, c8.w};
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = y_value(a4[q * 4 + e], acc[fm][fn][q * 4 + e] - a4[q * 4 + e], rs4 * cs4[e],
                                       rs8 * cs8[e]);
                    const int n = col0 + nl + q * 8;
                    _Float16 *dst = a.y + (int64_t)m * a.ldy + n;
                    if (m < a.M) {
                        if (vec_store && n + 3 < a.N) {
                            *reinterpret_cast<uint2 *>(dst) = uint2{pack_half2(v[0], v[1]), pack_half2(v[2], v[3])};
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < a.N)
                                    dst[e] = (_Float16)v[e];
                        }
                    }
                }
            }
        }
    }
}

// Epilogue of a tile that lies inside Y (rows 16-byte aligned), by halves of
// 64 columns, row block by row block. For each half of a row block, its two
// column blocks are finished (fp32 partial from the INT4 sums, the INT8 tail
// product, accumulated in place on top of the INT4 sums and recovered as
// the difference, y = fp16(acc4 * (sa4 * sw4 / 256) + acc8 * (sa8 * sw8))) and
// written to the wave's LDS staging area in the transposed accumulator
// layout; the 32 x 64 result is then read back row-major and stored with
// 16-byte stores, eight full 128-byte lines per store instruction. The
// staging area belongs to one wave, whose LDS operations complete in order,
// so it needs no barrier.
__device__ __forceinline__ void epilogue_interior(const GemmArgs &a, v16i (&acc)[FM][FN], unsigned char *lds,
                                                  const float *sS, int T4, int T8, int row0, int col0, int wm,
                                                  int wn, int li, int lh, int wave, int lane) {
    unsigned char *stg = lds + STAGES * STAGE + SCALE_BYTES + wave * STG_BYTES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // weight side of the tail for the two column blocks of this half; zero past the tail
        v4i pb8[2][MAX_TAIL_TILES][2];
#pragma unroll
        for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
            for (int j = 0; j < MAX_TAIL_TILES; ++j)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint4 p = *reinterpret_cast<const uint4 *>(lds + ((T4 + j) % STAGES) * STAGE + A_BYTES +
                                                                    swz(wn * WTN + (2 * h + f2) * 32 + li, 2 * s + lh));
                    pb8[f2][j][s] = j < T8 ? v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w} : v4i{0, 0, 0, 0};
                }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int ml = wm * WTM + fm * 32 + li;           // tile-local row of the lane
            const float rs4 = sS[ml] * (1.0f / 256.0f);
            const float rs8 = T8 > 0 ? sS[BM + ml] : 0.0f;    // tail scales are not loaded when T8 == 0
            v4i pa8[MAX_TAIL_TILES][2];
#pragma unroll
            for (int j = 0; j < MAX_TAIL_TILES; ++j)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint4 p = *reinterpret_cast<const uint4 *>(lds + ((T4 + j) % STAGES) * STAGE + swz(ml, 2 * s + lh));
                    pa8[j][s] = v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w};
                }
#pragma unroll
            for (int f2 = 0; f2 < 2; ++f2) {
                const int fn = 2 * h + f2;
                const int nl = wn * WTN + fn * 32 + lh * 4;   // tile-local first column of the lane
                // INT4 sums copied out (exact ints), then the tail product is
                // accumulated in place on top of them: acc8 = sum - acc4
                int a4[16];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    a4[r] = acc[fm][fn][r];
#pragma unroll
                for (int j = 0; j < MAX_TAIL_TILES; ++j)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(pb8[f2][j][s], pa8[j][s], acc[fm][fn], 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(sS + 2 * BM + nl + q * 8);
                    const float4 c8v = *reinterpret_cast<const float4 *>(sS + 3 * BM + nl + q * 8);
                    const float4 c8 = T8 > 0 ? c8v : float4{0.0f, 0.0f, 0.0f, 0.0f};
                    const float cs4[4] = {c4.x, c4.y, c4.z, c4.w}, cs8[4] = {c8.x, c8.y, c8.z, c8.w};
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = y_value(a4[q * 4 + e], acc[fm][fn][q * 4 + e] - a4[q * 4 + e], rs4 * cs4[e],
                                       rs8 * cs8[e]);
                    *reinterpret_cast<uint2 *>(stg + li * STG_PITCH + (f2 * 32 + q * 8 + lh * 4) * 2) =
                        uint2{pack_half2(v[0], v[1]), pack_half2(v[2], v[3])};
                }
            }
            // 32 x 64 staged: lane reads 16 bytes of row 8 i + lane / 8
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = i * 8 + (lane >> 3), c = lane & 7;
                const uint4 v = *reinterpret_cast<const uint4 *>(stg + r * STG_PITCH + c * 16);
                _Float16 *dst = a.y + (int64_t)(row0 + wm * WTM + fm * 32 + r) * a.ldy + col0 + wn * WTN + h * 64 + c * 8;
                *reinterpret_cast<uint4 *>(dst) = v;
            }
        }
    }
}

// One 256 x 256 output tile. `lds`: the ring of K-tiles, then the tile's
// scales (sa4 rows, sa8 rows, sw4 columns, sw8 columns).
template <bool EXPORT, bool INTERIOR>
__device__ __forceinline__ void gemm_big_tile(const GemmArgs &a, unsigned char *lds, int row0, int col0) {
    const float *sS = reinterpret_cast<const float *>(lds + STAGES * STAGE);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lh = lane >> 5;

    const int T4 = (int)(a.pitch4 / kTileBytes);   // INT4 K-tiles: ring tiles 0 .. T4-1
    const int T8 = (int)(a.pitch8 / kTileBytes);   // tail K-tiles: ring tiles T4 .. T-1
    const int T = T4 + T8;

    // ---- DMA sources of this lane (as in the 128 x 128 kernel) ------------------
    // Slot q = j * 256 + tid of a tile holds row q / 4 (of the activation or
    // weight quarter j), chunk (q % 4) ^ f(row): byte offsets for the INT4
    // and the INT8 tail operands, fixed for the whole K loop.
    static_assert(DA == 4 && DB == 4, "eight DMA instructions per tile");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t o4[8], o8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int q = (j & 3) * kThreads + tid;
        const uint32_t row = j < 4 ? min(row0 + (q >> 2), a.M - 1) : min(col0 + (q >> 2), a.N - 1);
        o4[j] = row * (uint32_t)a.pitch4 + dma_chunk_offset(q);
        o8[j] = row * (uint32_t)a.pitch8 + dma_chunk_offset(q);
    }
    // DMA instruction j (0..7) of ring tile tt: j < 4 a quarter of the
    // activation rows, j >= 4 of the weight rows (each wave moves its own 1 KB
    // of every quarter). Ring tiles past the tail reload the last INT4 tile
    // into their stage, which nothing reads again: every iteration of the K
    // loop then issues exactly one tile of DMA, with no branch.
    auto issue_part = [&](int tt, int j) {
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE + (j < 4 ? 0 : A_BYTES) + wave_u * 1024 +
                            (j & 3) * 4096;
        const bool tail = tt >= T4 && tt < T;
        const int t4 = tt < T4 ? tt : T4 - 1;
        const uint8_t *base = tail ? (j < 4 ? reinterpret_cast<const uint8_t *>(a.a8)
                                            : reinterpret_cast<const uint8_t *>(a.w8)) + (tt - T4) * kTileBytes
                                   : (j < 4 ? a.a4 : a.w4) + t4 * kTileBytes;
        dma16(base, tail ? o8[j] : o4[j], st);
    };
    auto issue = [&](int tt) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            issue_part(tt, j);
    };

    // ---- scales of the tile, ahead of every K-tile ---------------------------------
    // Issued first, so the wait for K-tile 0 covers them as well (loads
    // complete in order). Lane tid carries row row0 + tid and column col0 + tid.
    {
        const uint32_t ss = lds_addr(sS) + wave_u * 256;
        const int64_t mr = min(row0 + tid, a.M - 1), nc = min(col0 + tid, a.N - 1);
        dma4(a.sa4 + mr * a.G, ss);
        dma4(a.sw4 + nc * a.G, ss + 2 * BM * 4);
        if (T8 > 0) {
            dma4(a.sa8 + mr, ss + BM * 4);
            dma4(a.sw8 + nc, ss + 3 * BM * 4);
        }
    }

    // ---- main loop over the INT4 tiles ------------------------------------------------
    // Software pipeline, per wave: at the top of iteration t the registers hold
    // sub-step 0 of K-tile t widened (Wc) and sub-step 1 raw (R1). After the
    // barrier that makes K-tile t+1 visible, each sub-step's 32 MFMAs run in 8
    // chunks of four; a chunk also widens one fragment of the next sub-step,
    // reads fragments of K-tile t+1 from LDS (used eight chunks later) and, in
    // the first sub-step, issues one DMA instruction of K-tile t+4. Chunks are
    // scheduling barriers, so this order survives compilation. Every wave has
    // all its reads of tile t back (lgkmcnt 0) before the barrier, so tile t's
    // stage takes the DMA of tile t+4 after it: DMA runs three tiles ahead.
#pragma unroll
    for (int p = 0; p <= PREFETCH; ++p)
        issue(p);
    v16i acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[fm][fn][r] = 0;
    Frag R0, R1;
    Wide Wc, Wn;
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(PREFETCH * D));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    read_frag(R0, lds, 0, wm, wn, li, lh);
    read_frag(R1, lds, 1, wm, wn, li, lh);
    widen(Wc, R0);
    for (int tt = 0; tt < T4; ++tt) {
        compiler_fence();
        // K-tile tt+1 has landed: ring tiles up to tt + PREFETCH are issued
        // (prologue and one per iteration, past the tail included)
        __builtin_amdgcn_s_waitcnt(vmcnt_only((PREFETCH - 1) * D));
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));   // reads of K-tile tt are back
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        const int nt = tt + PREFETCH + 1;               // ring tile whose DMA this iteration issues
        // K-tile tt+1 (on the last iteration the first tail tile or a stale
        // stage: in bounds, and the values are never used)
        const unsigned char *nx = lds + ((tt + 1) % STAGES) * STAGE;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            issue_part(nt, i);
            mma_four(acc, Wc, i);
            widen_one(Wn, R1, i);
            const uint4 v = read_one(nx, i, 0, wm, wn, li, lh);
            if (i < 4)
                R0.a[i] = v;
            else
                R0.b[i - 4] = v;
            chunk_order<1>();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mma_four(acc, Wn, i);
            widen_one(Wc, R0, i);
            if (i < 4) {
#pragma unroll
                for (int k = 2 * i; k < 2 * i + 2; ++k) {
                    const uint4 v = read_one(nx, k, 1, wm, wn, li, lh);
                    if (k < 4)
                        R1.a[k] = v;
                    else
                        R1.b[k - 4] = v;
                }
            }
            if (i < 4)
                chunk_order<2>();
            else
                chunk_order<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- the tail ------------------------------------------------------------------------
    // Every tail tile was issued in the last iterations (the tail has at most
    // four tiles, PREFETCH + 1 ahead of the last INT4 tile); tail tile j sits in
    // stage (T4 + j) % STAGES.
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();

    if constexpr (INTERIOR && !EXPORT)
        epilogue_interior(a, acc, lds, sS, T4, T8, row0, col0, wm, wn, li, lh, wave, lane);
    else
        epilogue<EXPORT>(a, acc, lds, sS, T4, T8, row0, col0, wm, wn, li, lh);
}

// INTERIOR: every tile lies inside Y (M and N multiples of the tile) and Y
// rows are 16-byte aligned, so the epilogue stores with no guard. It is a
// separate kernel rather than a branch per tile: with both epilogues in one
// body the accumulator file overflows into scratch.
template <bool EXPORT, bool INTERIOR>
__global__ __launch_bounds__(kThreads) void gemm_big_kernel(GemmArgs a) {
    __shared__ __align__(16) unsigned char lds[LDS_BYTES];
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    gemm_big_tile<EXPORT, INTERIOR>(a, lds, tm * BM, tn * BN);
}

}  // namespace gemm_big_impl

using namespace gemm_big_impl;

bool gemm_big_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t G) {
    const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    // the tail is accumulated on top of the INT4 sums (16384 * (K_n + n_out) must fit int32)
    return G == 1 && K_n > 0 && w4a4_pitch8_bytes(n_out) / kTileBytes <= MAX_TAIL_TILES && tiles >= 256 &&
           (int64_t)(K_n + n_out) * 16384 < (int64_t)1 << 31;
}

hipError_t launch_gemm_big(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const bool interior = a.M % BM == 0 && a.N % BN == 0 && a.ldy % 8 == 0 &&
                          reinterpret_cast<uintptr_t>(a.y) % 16 == 0;
    if (export_acc)
        hipLaunchKernelGGL((gemm_big_kernel<true, false>), dim3(tiles), dim3(kThreads), 0, stream, a);
    else if (interior)
        hipLaunchKernelGGL((gemm_big_kernel<false, true>), dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_big_kernel<false, false>), dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
