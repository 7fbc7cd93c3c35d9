// GEMM for decode batches (M <= 128 tokens): the weights are streamed once
// from HBM.
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part with group
// quantization plus an 8-bit outlier part over reordered channels; Key points
// item 5: symmetric scales factor out of the integer sums) and the QUIK
// abstract (one-token decode is memory-bound).
//
// CDNA4 design (HBM-bound: every weight byte is read once). For M <= 32
// (gemm_decode_kernel<XI>; the row-block kernel further down takes 32 < M <= 128):
// * A workgroup owns 32 output columns and all M <= 32 token rows: one
//   32 x 32 block of v_mfma_i32_32x32x32_i8 with the weight fragment as the
//   first operand (lane (li, lh) holds token row li and the columns
//   8 (r / 4) + 4 lh + r % 4). Token rows past M repeat row M - 1; their
//   results are dropped.
// * Its eight waves split the INT4 K-tiles (64 bytes of every row, 128
//   channels) into contiguous ranges. Each wave moves pairs of tiles (128
//   bytes of each of the 32 weight rows and of the token rows, 8 XI of them
//   for a batch of at most 8 XI rows) into a two-slot
//   LDS ring of its own by direct global->LDS DMA, eight lanes per row, so
//   each DMA instruction covers eight whole cache lines; it reads them back
//   in MFMA layout (16-byte chunks XOR-swizzled by row, conflict-free).
// * Each INT4 tile is folded at once: y += float(acc) * (sa * sw / 256) with
//   the scale products from one v_mfma_f32_32x32x2_f32 (an outer product of
//   the column and the row scales in the accumulator layout); this holds for
//   any group size that is a multiple of 128 (a tile lies inside one group).
//   A wave's scales and first INT8 tail tile are requested just before its
//   first DMA. The INT8 tail is read directly, accumulated over its tiles and
//   folded once.
// * The eight partial blocks are added through LDS in wave order (the same
//   order in every call), then written as fp16.
#include <algorithm>
#include <type_traits>

#include "w4a4.h"
#include "gemm_common.h"

namespace w4a4 {
namespace gemm_decode_impl {

using namespace gemm_impl;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int BN = 32;                    // output columns per workgroup
constexpr int MAXM = 32;                  // token rows
constexpr int MAXT = 16;                  // INT4 tiles per wave (K_n <= 16384)
constexpr int PAIR = 128;                 // bytes of a row in a pair of tiles
constexpr int SLOT = 2 * 32 * PAIR;       // 32 weight rows, then 32 token rows
constexpr int WAVE_LDS = 2 * SLOT;        // two slots per wave
constexpr int RED_BYTES = WAVES * 16 * 64 * 4;
static_assert(WAVES * WAVE_LDS >= RED_BYTES, "the reduction reuses the ring");
constexpr int MAXG = MAXT * WAVES;        // scale groups of a row (K_n <= 16384, groups >= 128 channels)
constexpr int SC_BYTES = 32 * MAXG * 4;   // the stripe's 32 weight rows (or 32 token rows) of scales
constexpr int DECODE_LDS = WAVES * WAVE_LDS + 2 * SC_BYTES;

__device__ __forceinline__ v4i as_v4i(uint4 p) { return v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w}; }

// 16-byte chunk c of row r of a pair slot sits at chunk position c ^ (r & 7)
__device__ __forceinline__ int pair_off(int r, int c) { return r * PAIR + ((c ^ (r & 7)) << 4); }

// Accumulator export (test path): add the exact integer sums of one 32 x 32
// block (token rows m0 + li, columns n0 + 8 (e / 4) + 4 lh + e % 4) into the
// zeroed export slice `dst` [M, N]; the waves that share a scale group add
// their parts.
__device__ __forceinline__ void export_block(const v16i &acc, int32_t *dst, int shift, const GemmArgs &a, int m0,
                                             int n0, int li, int lh) {
    const int m = m0 + li;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int n = n0 + 8 * (e / 4) + 4 * lh + e % 4;
        if (m < a.M && n < a.N)
            export_add(dst + (int64_t)m * a.N + n, acc[e] >> shift);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    compiler_fence();
}

// XI: DMA instructions per pair for the token rows (eight rows each): rows
// past the batch are never stored, so a batch of at most 8 XI rows moves
// only its own rows (the MFMA lanes of the rows past them read slot bytes
// whose results are dropped).
template <int XI, bool EXPORT>
__global__ __launch_bounds__(THREADS) void gemm_decode_kernel(GemmArgs a) {
    static_assert(XI >= 1 && XI <= 4, "one to four token DMA instructions per pair");
    constexpr int PD = 4 + XI;                                // DMA instructions per pair
    __shared__ __align__(16) unsigned char lds[DECODE_LDS];

    const int tid = threadIdx.x;
    // the wave index is uniform, so the tile schedule is scalar code
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    const int n0 = blockIdx.x * BN;
    const int T4 = (int)(a.pitch4 / kTileBytes), T8 = (int)(a.pitch8 / kTileBytes);
    const int tiles_per_group = a.group > 0 ? a.group / 128 : max(T4, 1);
    const int per = (T4 + WAVES - 1) / WAVES;                 // <= MAXT (checked at launch)
    const int tb = min(wave * per, T4), te = min(tb + per, T4);
    const int nt = te - tb, np = (nt + 1) / 2;                // tiles and pairs of this wave

    // ---- the INT4 scales of the stripe's weight rows and of the token rows:
    // each is one contiguous run of rows x G floats, staged into LDS by DMA
    // of 4 bytes per lane (every lane issues the same count; past the end a
    // lane repeats the last float into a slot nothing reads), ahead of
    // everything else. Then the wave's first INT8 tail tile. The DMA waits
    // are counted by hand; loads complete in order, so the first wait on a
    // pair also covers these older loads, and they travel with the first pairs.
    const int64_t nrow = min(n0 + li, a.N - 1), mrow = min(li, a.M - 1);
    const int wrows = min(32, a.N - n0), xrows = min(32, a.M);
    float *sws = reinterpret_cast<float *>(lds + WAVES * WAVE_LDS);
    float *sas = reinterpret_cast<float *>(lds + WAVES * WAVE_LDS + SC_BYTES);
    {
        const int nw = wrows * a.G, nx = xrows * a.G;          // <= 32 MAXG floats each
        const float *wsrc = a.sw4 + (int64_t)n0 * a.G;
        for (int i = 0; i * THREADS < nw; ++i)
            dma4s(wsrc, 4u * (uint32_t)min(i * THREADS + tid, nw - 1), lds_addr(sws) + i * THREADS * 4 + wave * 256);
        for (int i = 0; i * THREADS < nx; ++i)
            dma4s(a.sa4, 4u * (uint32_t)min(i * THREADS + tid, nx - 1), lds_addr(sas) + i * THREADS * 4 + wave * 256);
    }
    const int swrow = (int)(nrow - n0) * a.G, sarow = (int)mrow * a.G;
    const uint8_t *w8row = reinterpret_cast<const uint8_t *>(a.w8) + nrow * a.pitch8 + 16 * lh;
    const uint8_t *x8row = reinterpret_cast<const uint8_t *>(a.a8) + mrow * a.pitch8 + 16 * lh;
    uint4 tw[2] = {}, tx[2] = {};
    if (T8 > wave) {
        tw[0] = *reinterpret_cast<const uint4 *>(w8row + wave * kTileBytes);
        tw[1] = *reinterpret_cast<const uint4 *>(w8row + wave * kTileBytes + 32);
        tx[0] = *reinterpret_cast<const uint4 *>(x8row + wave * kTileBytes);
        tx[1] = *reinterpret_cast<const uint4 *>(x8row + wave * kTileBytes + 32);
    }

    // ---- DMA of a pair of tiles: instruction i covers rows 8 i .. 8 i + 7, lane
    // q row 8 i + q / 8 and stored chunk q % 8 (logical chunk (q % 8) ^ (row & 7));
    // chunks 4..7 are the second tile, or the first again past the last tile
    uint32_t ow[4], ox[4], owd[4], oxd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3), c = (lane & 7) ^ (r & 7);
        const int64_t wr = min(n0 + r, a.N - 1), xr = min(r, a.M - 1);
        ow[i] = (uint32_t)(wr * a.pitch4) + 16 * c;
        ox[i] = (uint32_t)(xr * a.pitch4) + 16 * c;
        owd[i] = (uint32_t)(wr * a.pitch4) + 16 * (c & 3);
        oxd[i] = (uint32_t)(xr * a.pitch4) + 16 * (c & 3);
    }
    unsigned char *wl = lds + wave * WAVE_LDS;
    auto issue = [&](int j) {                                 // pair j into slot j % 2
        const int t0 = tb + 2 * j;
        const bool dup = t0 + 1 >= te;                        // odd last pair: no second tile
        const uint32_t st = lds_addr(wl + (j & 1) * SLOT);
        const uint8_t *W = a.w4 + t0 * kTileBytes, *X = a.a4 + t0 * kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(W, dup ? owd[i] : ow[i], st + i * 1024);
#pragma unroll
        for (int i = 0; i < XI; ++i)
            dma16(X, dup ? oxd[i] : ox[i], st + 32 * PAIR + i * 1024);
    };

    v16f y = {};
    const v16f zf = {};
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // tile h of the pair in slot `sl`, k-th tile of the wave
    auto tile = [&](const unsigned char *sl, int h, int k) {
        v16i acc;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 4 * h + 2 * s + lh;
            const uint4 pw = *reinterpret_cast<const uint4 *>(sl + pair_off(li, c));
            const uint4 px = *reinterpret_cast<const uint4 *>(sl + 32 * PAIR + pair_off(li, c));
            const v4i w0 = {(int)nib_lo(pw.x), (int)nib_hi(pw.x), (int)nib_lo(pw.y), (int)nib_hi(pw.y)};
            const v4i w1 = {(int)nib_lo(pw.z), (int)nib_hi(pw.z), (int)nib_lo(pw.w), (int)nib_hi(pw.w)};
            const v4i x0 = {(int)nib_lo(px.x), (int)nib_hi(px.x), (int)nib_lo(px.y), (int)nib_hi(px.y)};
            const v4i x1 = {(int)nib_lo(px.z), (int)nib_hi(px.z), (int)nib_lo(px.w), (int)nib_hi(px.w)};
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0, x0, s == 0 ? zi : acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1, x1, acc, 0, 0, 0);
        }
        if constexpr (EXPORT)
            export_block(acc, a.acc4_out + (int64_t)((tb + k) / tiles_per_group) * a.M * a.N, 8, a, 0, n0, li, lh);
        // scale products S[n][m] = sw[n] * sa[m] / 256 (the k = 1 lanes give zero)
        const int g = (tb + k) / tiles_per_group;
        const float swk = sws[swrow + g] * (1.0f / 256.0f), sak = sas[sarow + g];
        const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : swk, lh ? 0.0f : sak, zf, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            y[e] = __builtin_fmaf((float)acc[e], S[e], y[e]);
    };

    // ---- INT4 tiles: two pairs in flight; the loop is unrolled (the scales of
    // tile k sit in registers sw[k], sa[k])
    if (np > 0)
        issue(0);
    if (np > 1)
        issue(1);
    // every lane's scale DMAs (older than its pairs) have landed
    compiler_fence();
    if (np > 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * PD));
    else if (np == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(PD));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MAXT / 2; ++j) {
        if (j < np) {
            compiler_fence();
            if (j + 1 < np)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(PD));   // pair j + 1 may stay in flight
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            compiler_fence();
            const unsigned char *sl = wl + (j & 1) * SLOT;
            tile(sl, 0, 2 * j);
            if (2 * j + 1 < nt)
                tile(sl, 1, 2 * j + 1);
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));       // this slot's reads are back
            compiler_fence();
            if (j + 2 < np)
                issue(j + 2);
        }
    }

    // ---- INT8 tail: wave w takes tail tiles w, w + 8, ... (the first one is
    // already in registers; folded once) -------------------------------------------------
    if (T8 > wave) {
        v16i acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[0]), as_v4i(tx[0]), zi, 0, 0, 0);
        acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[1]), as_v4i(tx[1]), acc8, 0, 0, 0);
        for (int t = wave + WAVES; t < T8; t += WAVES) {
            const uint4 w0 = *reinterpret_cast<const uint4 *>(w8row + t * kTileBytes);
            const uint4 w1 = *reinterpret_cast<const uint4 *>(w8row + t * kTileBytes + 32);
            const uint4 x0 = *reinterpret_cast<const uint4 *>(x8row + t * kTileBytes);
            const uint4 x1 = *reinterpret_cast<const uint4 *>(x8row + t * kTileBytes + 32);
            acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(w0), as_v4i(x0), acc8, 0, 0, 0);
            acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(w1), as_v4i(x1), acc8, 0, 0, 0);
        }
        if constexpr (EXPORT)
            export_block(acc8, a.acc8_out, 0, a, 0, n0, li, lh);
        const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : a.sw8[nrow], lh ? 0.0f : a.sa8[mrow], zf,
                                                             0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            y[e] = __builtin_fmaf((float)acc8[e], S[e], y[e]);
    }

    // ---- the eight partial blocks, added in wave order (in the ring's LDS, once
    // every wave is done with its ring) ------------------------------------------------
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);              // [wave][register][lane]
#pragma unroll
    for (int e = 0; e < 16; ++e)
        red[(wave * 16 + e) * 64 + lane] = y[e];
    __syncthreads();
    // thread tid: lane tid % 64, registers 2 (tid / 64) and 2 (tid / 64) + 1
    // (two consecutive columns of one token row)
    {
        const int l = tid & 63, e0 = 2 * (tid >> 6);
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            v0 += red[(w * 16 + e0) * 64 + l];
            v1 += red[(w * 16 + e0 + 1) * 64 + l];
        }
        const int m = l & 31;
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

// Decode batches of 32 < M <= 32 MB token rows: the same column stripes and K
// ranges, with MB row blocks per wave. Every wave streams single K-tiles of
// its 32 weight rows and 32 MB token rows into a two-slot LDS ring of its own
// by direct DMA (a tile's 64-byte row segments, chunks swizzled as in the
// other GEMM kernels); every row segment crosses from L2 once. Row blocks go
// in pairs, side by side (one MFMA per block per k-step), and the scale
// products of a pair come from one v_mfma_f32_32x32x1_2b_f32 (block b in
// lanes 0-31, b + 1 in 32-63). All scales sit in registers, loaded before the
// first DMA, which bounds a wave's range to MAXT_ROWS tiles. The partial
// blocks are added through LDS in wave order, one row block at a time.
constexpr int MAXT_ROWS = 8;                              // K_n <= 8192

template <int MB>
struct RowsRing {
    static constexpr int ROWS = 32 + 32 * MB;             // weight rows, then token rows
    static constexpr int DMA = ROWS / 16;                 // DMA instructions per tile
    static constexpr int SLOT = ROWS * kTileBytes;
    static constexpr int WAVE = 2 * SLOT;
    static constexpr int BYTES = WAVES * WAVE > WAVES * 16 * 64 * 4 ? WAVES * WAVE : WAVES * 16 * 64 * 4;
};

template <int MB, bool EXPORT>
__global__ __launch_bounds__(THREADS) void gemm_decode_rows_kernel(GemmArgs a) {
    using R = RowsRing<MB>;
    __shared__ __align__(16) unsigned char lds[R::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    const int n0 = blockIdx.x * BN;
    const int T4 = (int)(a.pitch4 / kTileBytes), T8 = (int)(a.pitch8 / kTileBytes);
    const int tiles_per_group = a.group > 0 ? a.group / 128 : max(T4, 1);
    const int per = (T4 + WAVES - 1) / WAVES;             // <= MAXT_ROWS (checked at launch)
    const int tb = min(wave * per, T4), te = min(tb + per, T4);
    const int nt = te - tb;

    // ---- scales of this wave's tiles, before any DMA (the DMA waits count DMA only)
    const int64_t nrow = min(n0 + li, a.N - 1);
    int64_t mrow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        mrow[b] = min(32 * b + li, a.M - 1);
    float sw[MAXT_ROWS], sa[MAXT_ROWS][MB];
#pragma unroll
    for (int k = 0; k < MAXT_ROWS; ++k) {
        const int g = min(tb + k, T4 - 1) / tiles_per_group;
        sw[k] = a.sw4[nrow * a.G + g] * (1.0f / 256.0f);
#pragma unroll
        for (int b = 0; b < MB; ++b)
            sa[k][b] = a.sa4[mrow[b] * a.G + g];
    }
    // INT8 tail items (tile t, row block b), i = t MB + b, go to wave i % 8;
    // this wave's first item is requested here, with the scales (loads
    // complete in order: the first DMA wait covers them)
    const uint8_t *w8row = reinterpret_cast<const uint8_t *>(a.w8) + nrow * a.pitch8 + 16 * lh;
    auto x8ptr = [&](int i) {
        return reinterpret_cast<const uint8_t *>(a.a8) + min(32 * (i % MB) + li, a.M - 1) * (int64_t)a.pitch8 +
               16 * lh + (i / MB) * kTileBytes;
    };
    uint4 tw[2] = {}, tx[2] = {};
    if (T8 * MB > wave) {
        tw[0] = *reinterpret_cast<const uint4 *>(w8row + (wave / MB) * kTileBytes);
        tw[1] = *reinterpret_cast<const uint4 *>(w8row + (wave / MB) * kTileBytes + 32);
        tx[0] = *reinterpret_cast<const uint4 *>(x8ptr(wave));
        tx[1] = *reinterpret_cast<const uint4 *>(x8ptr(wave) + 32);
    }

    // ---- DMA of one tile: instruction i covers ring rows 16 i .. 16 i + 15, lane
    // q row 16 i + q / 4 and stored chunk q % 4 (see dma_chunk_offset)
    uint32_t voff[R::DMA];
#pragma unroll
    for (int i = 0; i < R::DMA; ++i) {
        const int r = 16 * i + (lane >> 2);
        const int64_t src = r < 32 ? min(n0 + r, a.N - 1) : min(r - 32, a.M - 1);
        voff[i] = (uint32_t)(src * a.pitch4) + dma_chunk_offset(r * 4 + (lane & 3));
    }
    unsigned char *wl = lds + wave * R::WAVE;
    // ring rows [16 I0, 16 I1) of tile tb + k into slot k % 2
    auto issue_rows = [&](int k, auto i0, auto i1) {
        const int t = tb + k;
        const uint32_t st = lds_addr(wl + (k & 1) * R::SLOT);
        const uint8_t *W = a.w4 + t * kTileBytes, *X = a.a4 + t * kTileBytes;
#pragma unroll
        for (int i = decltype(i0)::value; i < decltype(i1)::value; ++i)
            dma16(i < 2 ? W : X, voff[i], st + i * 1024);
    };
    auto issue = [&](int k) { issue_rows(k, std::integral_constant<int, 0>{}, std::integral_constant<int, R::DMA>{}); };

    v16f y[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        y[b] = v16f{};
    const v16f zf = {};
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // Tile k from slot k % 2, a pair of row blocks at a time: the rows of the
    // weights and of a pair are read into registers, then those ring rows take
    // their part of tile k + 2 at once, while this tile's MFMAs run.
    auto tile = [&](int k) {
        const unsigned char *sl = wl + (k & 1) * R::SLOT;
        v4i w[2][2];
#pragma unroll
        for (int b0 = 0; b0 < MB; b0 += 2) {
            constexpr int kPair = 2;
            const int nb = b0 + 1 < MB ? kPair : 1;
            uint4 pw[2], px[kPair][2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (b0 == 0)
                    pw[s] = *reinterpret_cast<const uint4 *>(sl + swz(li, 2 * s + lh));
#pragma unroll
                for (int i = 0; i < kPair; ++i)
                    if (i < nb)
                        px[i][s] = *reinterpret_cast<const uint4 *>(sl + swz(32 + 32 * (b0 + i) + li, 2 * s + lh));
            }
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));       // these ring rows are free again
            compiler_fence();
            if (k + 2 < nt) {
                // weights (ring rows 0..31) with the first pair; a pair's token rows
                // are ring rows 32 + 32 b0 .. 32 + 32 (b0 + nb) - 1
                if (b0 == 0)
                    issue_rows(k + 2, std::integral_constant<int, 0>{},
                               std::integral_constant<int, (MB >= 2 ? 6 : 4)>{});
                else if (b0 == 2)
                    issue_rows(k + 2, std::integral_constant<int, 6>{}, std::integral_constant<int, R::DMA>{});
            }
            if (b0 == 0)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    w[s][0] = v4i{(int)nib_lo(pw[s].x), (int)nib_hi(pw[s].x), (int)nib_lo(pw[s].y), (int)nib_hi(pw[s].y)};
                    w[s][1] = v4i{(int)nib_lo(pw[s].z), (int)nib_hi(pw[s].z), (int)nib_lo(pw[s].w), (int)nib_hi(pw[s].w)};
                }
            v4i x[kPair][2][2];
#pragma unroll
            for (int i = 0; i < kPair; ++i)
                if (i < nb)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const uint4 q = px[i][s];
                        x[i][s][0] = v4i{(int)nib_lo(q.x), (int)nib_hi(q.x), (int)nib_lo(q.y), (int)nib_hi(q.y)};
                        x[i][s][1] = v4i{(int)nib_lo(q.z), (int)nib_hi(q.z), (int)nib_lo(q.w), (int)nib_hi(q.w)};
                    }
            v16i acc[kPair];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < kPair; ++i)
                    if (i < nb)
                        acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[q >> 1][q & 1], x[i][q >> 1][q & 1],
                                                                       q == 0 ? zi : acc[i], 0, 0, 0);
            if constexpr (EXPORT) {
#pragma unroll
                for (int i = 0; i < kPair; ++i)
                    if (i < nb)
                        export_block(acc[i], a.acc4_out + (int64_t)((tb + k) / tiles_per_group) * a.M * a.N, 8, a,
                                     32 * (b0 + i), n0, li, lh);
            }
            // scale products one block at a time (16 registers live)
#pragma unroll
            for (int i = 0; i < kPair; ++i)
                if (i < nb) {
                    const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : sw[k], lh ? 0.0f : sa[k][b0 + i],
                                                                         zf, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        y[b0 + i][e] = __builtin_fmaf((float)acc[i][e], S[e], y[b0 + i][e]);
                }
        }
    };

    // ---- INT4 tiles: two in flight, the loop unrolled (scales in registers)
    if (nt > 0)
        issue(0);
    if (nt > 1)
        issue(1);
#pragma unroll
    for (int k = 0; k < MAXT_ROWS; ++k) {
        if (k < nt) {
            compiler_fence();
            if (k + 1 < nt)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(R::DMA));      // tile k + 1 may stay in flight
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            compiler_fence();
            tile(k);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    // ---- INT8 tail items of this wave (the first one already in registers)
    if (T8 * MB > wave) {
        const float sw8 = a.sw8[nrow];
        for (int i = wave; i < T8 * MB; i += WAVES) {
            const int t = i / MB, b = i % MB;
            if (i != wave) {
                tw[0] = *reinterpret_cast<const uint4 *>(w8row + t * kTileBytes);
                tw[1] = *reinterpret_cast<const uint4 *>(w8row + t * kTileBytes + 32);
                tx[0] = *reinterpret_cast<const uint4 *>(x8ptr(i));
                tx[1] = *reinterpret_cast<const uint4 *>(x8ptr(i) + 32);
            }
            v16i acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[0]), as_v4i(tx[0]), zi, 0, 0, 0);
            acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[1]), as_v4i(tx[1]), acc8, 0, 0, 0);
            if constexpr (EXPORT)
                export_block(acc8, a.acc8_out, 0, a, 32 * b, n0, li, lh);
            const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : sw8, lh ? 0.0f : a.sa8[min(32 * b + li, a.M - 1)],
                                                                 zf, 0, 0, 0);
            // the block index is uniform: select y[b] without indexing a register array
#pragma unroll
            for (int bb = 0; bb < MB; ++bb)
                if (bb == b)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        y[bb][e] = __builtin_fmaf((float)acc8[e], S[e], y[bb][e]);
        }
    }

    // ---- partial blocks added in wave order, one row block at a time
    float *red = reinterpret_cast<float *>(lds);              // [wave][register][lane]
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e)
            red[(wave * 16 + e) * 64 + lane] = y[b][e];
        __syncthreads();
        const int l = tid & 63, e0 = 2 * (tid >> 6);
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            v0 += red[(w * 16 + e0) * 64 + l];
            v1 += red[(w * 16 + e0 + 1) * 64 + l];
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

}  // namespace gemm_decode_impl

using namespace gemm_decode_impl;

bool gemm_decode_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group) {
    (void)n_out;
    const int T4 = (K_n + 127) / 128;
    const int per = (T4 + WAVES - 1) / WAVES;
    // DMA offsets are 32-bit: every packed operand row must start below 4 GiB
    const int64_t pitch4 = (int64_t)T4 * kTileBytes;
    if ((int64_t)N * pitch4 >= (int64_t(1) << 32) || (int64_t)M * pitch4 >= (int64_t(1) << 32))
        return false;
    return M >= 1 && K_n >= 128 && (group == 0 || group % 128 == 0) &&
           ((M <= MAXM && per <= MAXT) || (M <= 4 * MAXM && per <= MAXT_ROWS));
}

const char *decode_kernel_name(int rows) {
    switch ((rows + MAXM - 1) / MAXM) {
    case 1:
        switch ((rows + 7) / 8) {
        case 1: return "gemm_decode_kernel<1, false>";
        case 2: return "gemm_decode_kernel<2, false>";
        case 3: return "gemm_decode_kernel<3, false>";
        default: return "gemm_decode_kernel<4, false>";
        }
    case 2: return "gemm_decode_rows_kernel<2, false>";
    case 3: return "gemm_decode_rows_kernel<3, false>";
    default: return "gemm_decode_rows_kernel<4, false>";
    }
}

template <bool EXPORT>
static void launch_decode(const GemmArgs &a, hipStream_t stream) {
    const int blocks = (a.N + BN - 1) / BN;
    const int mb = (a.M + MAXM - 1) / MAXM;
    if (mb <= 1) {
        const int xi = (a.M + 7) / 8;
        if (xi <= 1)
            hipLaunchKernelGGL((gemm_decode_kernel<1, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
        else if (xi == 2)
            hipLaunchKernelGGL((gemm_decode_kernel<2, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
        else if (xi == 3)
            hipLaunchKernelGGL((gemm_decode_kernel<3, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<4, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
    }
    else if (mb == 2)
        hipLaunchKernelGGL((gemm_decode_rows_kernel<2, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
    else if (mb == 3)
        hipLaunchKernelGGL((gemm_decode_rows_kernel<3, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_decode_rows_kernel<4, EXPORT>), dim3(blocks), dim3(THREADS), 0, stream, a);
}

hipError_t launch_gemm_decode(const GemmArgs &a, bool export_acc, hipStream_t stream) {
    if (export_acc)
        launch_decode<true>(a, stream);
    else
        launch_decode<false>(a, stream);
    return hipGetLastError();
}

}  // namespace w4a4
