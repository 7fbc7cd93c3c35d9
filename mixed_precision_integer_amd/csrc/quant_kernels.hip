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
// * Persistent workgroups loop over rows. Rows stream in by direct
//   global->LDS DMA (16 bytes per lane, non-temporal: each row is read once),
//   double buffered: the first two rows
//   are requested at once, then each next row's DMA is in flight while the
//   current row is quantized. LDS holds only the two row buffers and small
//   reduction tables, sized statically per row-length bucket (K <= 4096,
//   8192, 16384, 24576); long rows use more lanes per workgroup. Up to 512
//   lanes the kernel is held to 64 VGPRs so that every workgroup the
//   occupancy query counts is resident from the start.
// * The channels a lane handles are the same in every row, so the
//   permutation entries it needs are loaded once per workgroup into
//   registers (uint16 pairs); the per-row gather is then one LDS read per
//   channel with no dependent index load.
// * Two barriers per row: one after the row has landed, one after the
//   absmax reductions; every lane then derives the scale and reciprocal it
//   needs itself (identical arithmetic in every lane, so identical values).
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
#include <atomic>
#include <type_traits>

#include "quant_internal.h"

namespace w4a4 {
namespace quant_impl {

typedef _Float16 half2 __attribute__((ext_vector_type(2)));

constexpr int kMaxDevices = 64;

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

__device__ __forceinline__ _Float16 lo_half(uint32_t p) { return __builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFF)); }
__device__ __forceinline__ _Float16 hi_half(uint32_t p) { return __builtin_bit_cast(_Float16, (uint16_t)(p >> 16)); }

__device__ __forceinline__ float recip_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// x^2 * 2^48 of an fp16 value, exactly, as an integer below 2^80: with
// x = Mx * 2^(sh - 24) (Mx the significand with its hidden bit, sh = 0 for
// subnormals), x^2 * 2^48 = Mx^2 * 2^(2 sh).
__device__ __forceinline__ unsigned __int128 square_q48(uint32_t h) {
    const uint32_t e = (h >> 10) & 31, m = h & 1023;
    const uint32_t mx = e ? (m | 1024u) : m, sh = e ? e - 1 : 0;
    return (unsigned __int128)(mx * mx) << (2 * sh);
}

__device__ __forceinline__ unsigned __int128 wave_sum_u128(unsigned __int128 s) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)__shfl_xor((int)(uint32_t)(s >> (32 * k)), off, 64);
        s += (unsigned __int128)w[0] | ((unsigned __int128)w[1] << 32) | ((unsigned __int128)w[2] << 64) |
             ((unsigned __int128)w[3] << 96);
    }
    return s;
}

// RMSNorm of two packed fp16 values: fl16(gamma * fl16(fl32(x * rstd))). The
// product of two fp16 values is exact in fp32, so the packed fp16 multiply
// rounds it once, like the fp16 model does.
__device__ __forceinline__ uint32_t norm_pair(uint32_t xv, uint32_t g, float rstd) {
#pragma clang fp contract(off)
    const float p0 = (float)lo_half(xv) * rstd, p1 = (float)hi_half(xv) * rstd;
    const half2 h = {(_Float16)p0, (_Float16)p1};
    return __builtin_bit_cast(uint32_t, h * __builtin_bit_cast(half2, g));
}

// The row DMA of dma16 with the non-temporal cache policy: every X row is read
// exactly once, so it streams past the caches. (Measured 5-12% faster on the
// producer; the GEMMs keep cached DMA, which their tile reuse needs.)
__device__ __forceinline__ void dma16_stream(const void *base, uint32_t voff, uint32_t lds) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sb), "s"(sl)
                 : "memory", "m0");
}

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

// u6 operand of the FP6 GEMM: rows in blocks of 32 and channels in tiles of
// 64 (two 32-channel chunks); the block of row block b and tile t is 1536
// bytes at (b * T + t) * 1536, T = pitch4 / 32. Each chunk of a row is a
// 192-bit image holding the code of channel i at bits 6i; image bytes 0..15
// of row r's chunk h sit at 512 h + 16 r of the block, bytes 16..23 at
// 1024 + 256 h + 8 r.
constexpr int64_t kU6Block = 1536;

// E2M3 codes of q / 8 for four offset codes c = q + 8 (bytes, 0..15): two
// 8-entry byte tables (c < 8 and c >= 8) looked up by v_perm with c & 7,
// then a third v_perm takes each byte from the second table where bit 3 of
// c is set. Tables (the code is |q| with the sign in bit 5): q = -8..-1 ->
// 40 39 38 37 36 35 34 33; q = 0..7 -> 0 1 2 3 4 5 6 7.
__device__ __forceinline__ uint32_t e2m3_of_offset4(uint32_t c) {
    const uint32_t sel = c & 0x07070707u;
    const uint32_t neg = __builtin_amdgcn_perm(0x21222324u, 0x25262728u, sel);
    const uint32_t pos = __builtin_amdgcn_perm(0x07060504u, 0x03020100u, sel);
    return __builtin_amdgcn_perm(pos, neg, ((c >> 1) & 0x04040404u) | 0x03020100u);
}

// Four 6-bit codes in the low bits of four bytes -> 24 contiguous bits.
__device__ __forceinline__ uint32_t pack6x4(uint32_t x) {
    const uint32_t v = (x & 0x003F003Fu) | ((x >> 2) & 0x0FC00FC0u);   // fields at bits 0, 6, 16, 22
    return (v & 0xFFFu) | ((v >> 4) & 0xFFF000u);
}

// The value of `v` in lane SRC (0..3) of this lane's quad.
template <int SRC>
__device__ __forceinline__ uint32_t quad_read(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, SRC * 0x55, 0xF, 0xF, false);   // quad_perm [SRC x 4]
}

// Maxima of non-negative floats as unsigned integers (their bit patterns
// order the same way; no NaN canonicalization): DPP reads of another lane of
// the same row (dpp_ctrl CTRL).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// Maximum over the wave of values that are already equal within each quad
// (every lane gets it): two mirrors finish the rows of 16, readlane the wave.
__device__ __forceinline__ uint32_t wave_max_of_quads(uint32_t v) {
    v = dpp_max_u32<0x141>(v);                   // row_half_mirror: quads 0 <-> 1 of 8 lanes
    v = dpp_max_u32<0x140>(v);                   // row_mirror: halves of a row of 16
    const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
    v = dpp_max_u32<0xB1>(v);
    v = dpp_max_u32<0x4E>(v);
    return wave_max_of_quads(v);
}

// fl32(a / d) for a non-negative fp16 value a and d = 7 or 127, from
// r = fl32(1 / d): the same correction as exact_quotient, checked exhaustively
// against the correctly rounded quotient for every finite fp16 a (an infinite
// a keeps the division's infinite scale).
__device__ __forceinline__ float div_small_const(float a, float d, float r) {
#pragma clang fp contract(off)
    const float q0 = a * r;
    const float e = __builtin_fmaf(-q0, d, a);
    const float q = __builtin_fmaf(e, r, q0);
    return a == __builtin_inff() ? a : q;
}

// exact_quotient of an fp16 value (the conversion folds into the FMAs)
__device__ __forceinline__ float exact_quotient_h(_Float16 x, float s, float r) {
#pragma clang fp contract(off)
    const float xf = (float)x;
    const float q0 = __builtin_fmaf(xf, r, 0.0f);
    const float e = __builtin_fmaf(-q0, s, xf);
    return __builtin_fmaf(e, r, q0);
}

// Store the 48 bits of head unit u (channels 8u .. 8u + 7, code i at bit 6i)
// of row rr of a row block into their place in the chunk image: unit p = u % 4
// of chunk h = (u / 4) % 2 of tile u / 8 covers image bytes 6p .. 6p + 5,
// written as one 4-byte and one 2-byte store (both aligned).
__device__ __forceinline__ void store_u6_unit(unsigned char *blocks, int u, int rr, uint64_t img) {
    const int p = u & 3, h = (u >> 2) & 1;
    unsigned char *blk = blocks + (int64_t)(u >> 3) * kU6Block;
    unsigned char *lo = blk + 512 * h + 16 * rr, *hi = blk + 1024 + 256 * h + 8 * rr;
    const uint32_t w0 = (uint32_t)img, w1 = (uint32_t)(img >> 32);
    const bool odd = p & 1;
    // 4-byte part: bytes 0..3 (p 0), 8..11 (p 1), 12..15 (p 2), hi 4..7 (p 3)
    unsigned char *d4 = p == 0 ? lo : p == 1 ? lo + 8 : p == 2 ? lo + 12 : hi + 4;
    // 2-byte part: bytes 4..5 (p 0), 6..7 (p 1), hi 0..1 (p 2), hi 2..3 (p 3)
    unsigned char *d2 = p == 0 ? lo + 4 : p == 1 ? lo + 6 : p == 2 ? hi : hi + 2;
    *reinterpret_cast<uint32_t *>(d4) = odd ? (w0 >> 16) | (w1 << 16) : w0;
    *reinterpret_cast<uint16_t *>(d2) = (uint16_t)(odd ? w0 : w1);
}

// Static LDS for rows of up to KMAX channels: two row buffers (whole DMA
// rounds), the group maxima of two consecutive rows and the wave maxima.
template <int KMAX, int THREADS>
struct RowLds {
    static constexpr int ROUND = THREADS * 16;   // bytes one DMA instruction moves per workgroup
    static constexpr int XB = (KMAX * 2 + ROUND - 1) / ROUND * ROUND;
    static constexpr int GMAX = KMAX / 128;
    unsigned char x[2][XB];
    unsigned gmax[2][GMAX];
    float red_h[2][THREADS / 64], red_t[2][THREADS / 64];
    uint32_t red_q[2][THREADS / 64][4];   // sums of squares per wave (RMSNorm)
};

// WIDE_TAIL: the outlier tail may need more than one 4-channel word per lane.
// Up to 512 lanes a workgroup is register-limited: 64 VGPRs (eight waves per
// SIMD) keep every workgroup the occupancy query counts resident at once;
// the FULL layout takes up to 84 VGPRs (six waves per SIMD), which measured
// faster than spilling at 64.
//
// NORM: the row is RMS-normalized first (the norm that precedes the layer,
// fused so that its fp16 output never goes to memory). The lane's gathered
// values cover every channel once, so the sum of squares comes from them:
// exact, as a 128-bit integer of x^2 * 2^48 terms (below 2^95 for K <= 2^15),
// reduced over the wave by shuffles and over the workgroup through LDS (a
// third barrier per row). Every lane then derives
// rstd = fl32(1 / sqrt(fl64(fl64(S) / K) + eps)) with correctly rounded binary64
// operations, normalizes its values in registers and only then takes the
// absmax. The norm weights of the lane's channels are gathered once per
// workgroup, like the permutation.
//
// FULL: K and K_n are multiples of 8 (so n_out is too) and the tail fits one
// word per lane: every head unit and tail word lies wholly inside the row,
// so no entry needs a bounds check of its own. One mask per unit replaces
// the per-channel conditions, whose exec masks would otherwise stay live
// across the row loop and spill.
template <int KMAX, int THREADS, bool GROUPED, bool WIDE_TAIL, bool NORM, bool FULL, bool U6>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(THREADS <= 512 && !WIDE_TAIL && !NORM ? (FULL ? 6 : 8) : 4)))
void quant_rows_kernel(QuantArgs a) {
    static_assert(!(FULL && WIDE_TAIL), "a full-row layout has one tail word per lane");
    using L = RowLds<KMAX, THREADS>;
    constexpr int NW = THREADS / 64;
    constexpr int UMAX = (KMAX / 8 + THREADS - 1) / THREADS;    // head units (8 channels) per lane
    constexpr int TW = WIDE_TAIL ? (KMAX / 4 + THREADS - 1) / THREADS : 1;   // tail words per lane
    __shared__ __align__(16) L sm;

    const int K = a.K, K_n = a.K_n, n_out = a.n_out, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);

    const int nfull = K / 8;                       // whole 16-byte chunks of a row
    const int rounds = (nfull + THREADS - 1) / THREADS;
    auto issue_row = [&](int row, int b) {
        const unsigned char *src = reinterpret_cast<const unsigned char *>(a.src + (int64_t)row * a.ld);
        const uint32_t d = lds_addr(sm.x[b]) + wave_u * 1024;
        for (int j = 0; j < rounds; ++j) {
            const int c = j * THREADS + tid;
            dma16_stream(src, (uint32_t)(c < nfull ? c : 0) * 16, d + j * L::ROUND);
        }
    };

    const int U = (K_n + 7) / 8;
    const int W4 = (int)(a.pitch4 / 4), W8 = (int)(a.pitch8 / 4);

    // First row of this workgroup. For the u6 head, the rows that are in
    // flight together on one XCD are consecutive: workgroups are handed to
    // the eight XCDs in turn, so workgroup w takes the place (w % 8) P + w / 8
    // (P = grid / 8), and a 32-row block's partial-line stores meet in one
    // L2 instead of being written back piecewise from eight.
    int row = blockIdx.x;
    if (U6 && gridDim.x % 8 == 0)
        row = (int)((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8);
    if (row < a.rows)
        issue_row(row, 0);
    if (row + (int)gridDim.x < a.rows)         // the second row streams in at once as well
        issue_row(row + gridDim.x, 1);

    // The channels a lane reads are the same in every row, so their source
    // positions (the permutation) are loaded once into registers as uint16
    // pairs: head unit u = i * THREADS + tid holds reordered channels 8u..8u+7,
    // tail word w = i * THREADS + tid holds K_n + 4w .. K_n + 4w + 3. All loads
    // are issued (indices clamped into the array) before any is waited for.
    uint32_t pv[UMAX][4], pt[TW][2];
    {
        // 16-byte loads (a head unit's 8 entries are two of them; a tail word
        // is one when K_n % 4 == 0), index clamped into the array; entries
        // past the last whole int4 are fixed up with scalar loads after.
        // (a null permutation is the identity order)
        const int K4 = K / 4;
        const int4 *perm4 = reinterpret_cast<const int4 *>(a.perm);
        auto entry4 = [&](int q) { return perm4 ? perm4[q] : int4{4 * q, 4 * q + 1, 4 * q + 2, 4 * q + 3}; };
        int4 e[UMAX][2], f[TW];
        if (K4 > 0) {
#pragma unroll
            for (int i = 0; i < UMAX; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    e[i][h] = entry4(min(2 * (i * THREADS + tid) + h, K4 - 1));
#pragma unroll
            for (int i = 0; i < TW; ++i)
                f[i] = entry4(min(K_n / 4 + i * THREADS + tid, K4 - 1));
        } else {                                   // K < 4: every entry comes from fix() below
#pragma unroll
            for (int i = 0; i < UMAX; ++i)
                e[i][0] = e[i][1] = int4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < TW; ++i)
                f[i] = int4{0, 0, 0, 0};
        }
        const bool tail4 = (K_n & 3) == 0;
        auto entry = [&](int j) { return a.perm ? a.perm[j] : j; };
        auto fix = [&](int v, int j) { return (!FULL && j >= 4 * K4 && j < K) ? entry(j) : v; };
        auto pack = [](int lo, int hi) { return (uint32_t)(lo & 0xFFFF) | ((uint32_t)hi << 16); };
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int j0 = (i * THREADS + tid) * 8;
            pv[i][0] = pack(fix(e[i][0].x, j0), fix(e[i][0].y, j0 + 1));
            pv[i][1] = pack(fix(e[i][0].z, j0 + 2), fix(e[i][0].w, j0 + 3));
            pv[i][2] = pack(fix(e[i][1].x, j0 + 4), fix(e[i][1].y, j0 + 5));
            pv[i][3] = pack(fix(e[i][1].z, j0 + 6), fix(e[i][1].w, j0 + 7));
        }
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int j0 = K_n + (i * THREADS + tid) * 4;
            if (FULL || tail4) {
                pt[i][0] = pack(fix(f[i].x, j0), fix(f[i].y, j0 + 1));
                pt[i][1] = pack(fix(f[i].z, j0 + 2), fix(f[i].w, j0 + 3));
            } else {
                pt[i][0] = pack(j0 < K ? entry(j0) : 0, j0 + 1 < K ? entry(j0 + 1) : 0);
                pt[i][1] = pack(j0 + 2 < K ? entry(j0 + 2) : 0, j0 + 3 < K ? entry(j0 + 3) : 0);
            }
        }
    }
    // norm weights of the lane's channels (indices clamped into the row)
    uint32_t gv[NORM ? UMAX : 1][4], gt[NORM ? TW : 1][2];
    if constexpr (NORM) {
        const uint16_t *gp = reinterpret_cast<const uint16_t *>(a.gamma);
        const uint32_t last = (uint32_t)K - 1;
        auto g2 = [&](uint32_t p) {
            return (uint32_t)gp[min(p & 0xFFFF, last)] | ((uint32_t)gp[min(p >> 16, last)] << 16);
        };
#pragma unroll
        for (int i = 0; i < UMAX; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                gv[i][k] = g2(pv[i][k]);
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int k = 0; k < 2; ++k)
                gt[i][k] = g2(pt[i][k]);
    }
    if (GROUPED)
        for (int t = tid; t < 2 * L::GMAX; t += THREADS)
            (&sm.gmax[0][0])[t] = 0u;

    for (int it = 0; row < a.rows; ++it, row += gridDim.x) {
        const int buf = it & 1;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(sm.x[buf]);
        unsigned *gm = sm.gmax[buf];
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
        if (it > 0 && row + (int)gridDim.x < a.rows)   // buffer buf ^ 1 held the previous row
            issue_row(row + gridDim.x, buf ^ 1);
        if (GROUPED)                               // the next row accumulates in the other table
            for (int t = tid; t < G; t += THREADS)
                sm.gmax[buf ^ 1][t] = 0u;

        // (2) gather head units and tail words into registers; absmax (packed fp16)
        uint32_t v[UMAX][4], tv[TW][2];
        float hmax = 0.0f, tmax = 0.0f;
        auto head_absmax = [&](int i) {
            const int u = i * THREADS + tid;
            const int j0 = u * 8;
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
        };
        auto tail_absmax = [&](int i) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const half2 h = __builtin_bit_cast(half2, tv[i][k] & 0x7FFF7FFFu);
                tmax = fmaxf(tmax, fmaxf((float)h.x, (float)h.y));
            }
        };
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = i * THREADS + tid;
            const int j0 = u * 8;
            if constexpr (FULL) {                  // entries are valid row positions even past U
                const uint32_t keep = u < U ? 0xFFFFFFFFu : 0u;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[i][k] = ((uint32_t)xs[pv[i][k] & 0xFFFF] | ((uint32_t)xs[pv[i][k] >> 16] << 16)) & keep;
            } else if (u < U && j0 + 8 <= K_n) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[i][k] = (uint32_t)xs[pv[i][k] & 0xFFFF] | ((uint32_t)xs[pv[i][k] >> 16] << 16);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = j0 + 2 * k;
                    const uint32_t lo = (u < U && j < K_n) ? xs[pv[i][k] & 0xFFFF] : 0u;
                    const uint32_t hi = (u < U && j + 1 < K_n) ? xs[pv[i][k] >> 16] : 0u;
                    v[i][k] = lo | (hi << 16);
                }
            }
            if (!NORM)
                head_absmax(i);
        }
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int w = i * THREADS + tid;
            if constexpr (FULL) {
                const uint32_t keep = 4 * w < n_out ? 0xFFFFFFFFu : 0u;
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    tv[i][k] = ((uint32_t)xs[pt[i][k] & 0xFFFF] | ((uint32_t)xs[pt[i][k] >> 16] << 16)) & keep;
            } else {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int j = K_n + 4 * w + 2 * k;
                    const uint32_t lo = j < K ? xs[pt[i][k] & 0xFFFF] : 0u;
                    const uint32_t hi = j + 1 < K ? xs[pt[i][k] >> 16] : 0u;
                    tv[i][k] = lo | (hi << 16);
                }
            }
            if (!NORM)
                tail_absmax(i);
        }
        if constexpr (NORM) {
            // (2n) exact sum of squares (zeros past the row's end add nothing),
            // rstd, then the normalized values and their absmax
            unsigned __int128 ss = 0;
#pragma unroll
            for (int i = 0; i < UMAX; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    ss += square_q48(v[i][k] & 0xFFFF) + square_q48(v[i][k] >> 16);
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    ss += square_q48(tv[i][k] & 0xFFFF) + square_q48(tv[i][k] >> 16);
            ss = wave_sum_u128(ss);
            if (lane == 0)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    sm.red_q[buf][wave][k] = (uint32_t)(ss >> (32 * k));
            lds_barrier();
            unsigned __int128 S = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                S += (unsigned __int128)sm.red_q[buf][w][0] | ((unsigned __int128)sm.red_q[buf][w][1] << 32) |
                     ((unsigned __int128)sm.red_q[buf][w][2] << 64) | ((unsigned __int128)sm.red_q[buf][w][3] << 96);
            const double var = (double)S * 0x1p-48 / (double)K + (double)a.eps;
            const float rstd = var == 0.0 ? 0.0f : (float)(1.0 / __builtin_sqrt(var));
            if (tid == 0 && a.rstd)
                a.rstd[row] = rstd;
#pragma unroll
            for (int i = 0; i < UMAX; ++i) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[i][k] = norm_pair(v[i][k], gv[i][k], rstd);
                head_absmax(i);
            }
#pragma unroll
            for (int i = 0; i < TW; ++i) {
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    tv[i][k] = norm_pair(tv[i][k], gt[i][k], rstd);
                tail_absmax(i);
            }
        }
        if (!GROUPED)
            hmax = wave_max(hmax);
        tmax = wave_max(tmax);
        if (lane == 0) {
            sm.red_h[buf][wave] = hmax;
            sm.red_t[buf][wave] = tmax;
        }
        lds_barrier();

        // (3) scales: every lane derives the ones it needs (identical values)
        float ra = 0.0f, ta = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            ra = fmaxf(ra, sm.red_h[buf][w]);
            ta = fmaxf(ta, sm.red_t[buf][w]);
        }
        const float s_row = ra / 7.0f, r_row = recip_or_zero(s_row);
        const float s8 = ta / 127.0f, r8 = recip_or_zero(s8);
        if (tid == 0) {
            if (!GROUPED && G > 0)
                a.s4[row] = s_row;
            if (a.s8)
                a.s8[row] = n_out > 0 ? s8 : 0.0f;
        }

        // (4) INT4 head: codes + 8 as bytes, even channels in one dword and odd
        //     ones in another, then one nibble interleave and an xor with 8
        //     (or, for the u6 operand, the FP6 E2M3 codes of q / 8)
        if constexpr (U6) {
            // The four units of a 32-channel chunk sit in one quad of lanes
            // (units i * THREADS + tid, THREADS and W4 multiples of 4): each
            // lane forms its unit's 48 bits, lane 0 of the quad collects the
            // other three by DPP and stores the chunk image as 16 + 8 bytes.
            // Units from U up to W4 hold zeros, i.e. code 0.
            const int64_t T6 = a.pitch4 / 32;
            unsigned char *blocks = a.u6 + (int64_t)(row >> 5) * T6 * kU6Block + 16 * (row & 31);
#pragma unroll
            for (int i = 0; i < UMAX; ++i) {
                const int u = i * THREADS + tid;
                if (u < W4) {                      // uniform over each quad
                    float sc = s_row, rc = r_row;
                    if (GROUPED && u < U) {
                        const int t = (u * 8) / a.group;
                        sc = __uint_as_float(gm[t]) / 7.0f;
                        rc = recip_or_zero(sc);
                        if ((u * 8) % a.group == 0)    // the group's first unit stores its scale
                            a.s4[(int64_t)row * G + t] = sc;
                    }
                    uint32_t c[2] = {0u, 0u};      // offset codes q + 8, elements 0..3 and 4..7
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float q0 = __builtin_rintf(exact_quotient((float)lo_half(v[i][k]), sc, rc)) + 8.0f;
                        const float q1 = __builtin_rintf(exact_quotient((float)hi_half(v[i][k]), sc, rc)) + 8.0f;
                        c[k >> 1] = __builtin_amdgcn_cvt_pk_u8_f32(q0, 2 * (k & 1), c[k >> 1]);
                        c[k >> 1] = __builtin_amdgcn_cvt_pk_u8_f32(q1, 2 * (k & 1) + 1, c[k >> 1]);
                    }
                    const uint32_t y0 = pack6x4(e2m3_of_offset4(c[0])), y1 = pack6x4(e2m3_of_offset4(c[1]));
                    const uint32_t w0 = y0 | (y1 << 24), w1 = y1 >> 8;
                    const uint32_t a1 = quad_read<1>(w0), b1 = quad_read<1>(w1);
                    const uint32_t a2 = quad_read<2>(w0), b2 = quad_read<2>(w1);
                    const uint32_t a3 = quad_read<3>(w0), b3 = quad_read<3>(w1);
                    if ((tid & 3) == 0) {
                        unsigned char *blk = blocks + (int64_t)(u >> 3) * kU6Block;
                        const int h = (u >> 2) & 1;
                        // image bytes 0..15: unit 0, unit 1, the first four bytes of unit 2
                        *reinterpret_cast<uint4 *>(blk + 512 * h) =
                            uint4{w0, __builtin_amdgcn_perm(a1, w1, 0x05040100u),
                                  __builtin_amdgcn_perm(b1, a1, 0x05040302u), a2};
                        // bytes 16..23: the last two bytes of unit 2, unit 3
                        *reinterpret_cast<uint2 *>(blk + 1024 + 256 * h - 8 * (row & 31)) =
                            uint2{__builtin_amdgcn_perm(a3, b2, 0x05040100u), __builtin_amdgcn_perm(b3, a3, 0x05040302u)};
                    }
                }
            }
        } else {
        uint32_t *q4row = reinterpret_cast<uint32_t *>(a.q4 + (int64_t)row * a.pitch4);
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = i * THREADS + tid;
            if (u < U) {
                float sc = s_row, rc = r_row;
                if (GROUPED) {
                    const int t = (u * 8) / a.group;
                    sc = __uint_as_float(gm[t]) / 7.0f;
                    rc = recip_or_zero(sc);
                    if ((u * 8) % a.group == 0)    // the group's first unit stores its scale
                        a.s4[(int64_t)row * G + t] = sc;
                }
                uint32_t ev = 0, od = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float c0 = __builtin_rintf(exact_quotient((float)lo_half(v[i][k]), sc, rc)) + 8.0f;
                    const float c1 = __builtin_rintf(exact_quotient((float)hi_half(v[i][k]), sc, rc)) + 8.0f;
                    ev = __builtin_amdgcn_cvt_pk_u8_f32(c0, k, ev);
                    od = __builtin_amdgcn_cvt_pk_u8_f32(c1, k, od);
                }
                q4row[u] = (ev | (od << 4)) ^ 0x88888888u;
            }
        }
        for (int u = U + tid; u < W4; u += THREADS)   // zero padding of the row pitch
            q4row[u] = 0u;
        }

        // (5) INT8 tail: 4 codes -> one dword (zero past the last outlier)
        if (a.q8) {
            uint32_t *q8row = reinterpret_cast<uint32_t *>(a.q8 + (int64_t)row * a.pitch8);
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                const int w = i * THREADS + tid;
                if (w < W8) {
                    uint32_t word = 0;
                    if (!FULL || 4 * w < n_out) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int j = K_n + 4 * w + k;
                            if (FULL || j < K) {
                                const uint32_t h = (k & 1) ? (tv[i][k >> 1] >> 16) : (tv[i][k >> 1] & 0xFFFF);
                                const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
                                const int q = (int)__builtin_rintf(exact_quotient(x, s8, r8));
                                word |= (uint32_t)(q & 0xFF) << (8 * k);
                            }
                        }
                    }
                    q8row[w] = word;
                }
            }
        }
    }
    if constexpr (U6) {
        // rows past the last one, up to the end of its 32-row block: code 0
        const int64_t T6 = a.pitch4 / 32;
        const int rows_padded = (a.rows + 31) & ~31;
        for (int zr = a.rows + (int)blockIdx.x; zr < rows_padded; zr += (int)gridDim.x) {
            unsigned char *blocks = a.u6 + (int64_t)(zr >> 5) * T6 * kU6Block;
            for (int u = tid; u < W4; u += THREADS)
                store_u6_unit(blocks, u, zr & 31, 0);
        }
    }
}

// Group scales (group of 128, 256, 512 or 64 * 8 * UPL channels, dividing a
// chunk): waves are independent
// workers, with no LDS and no barrier. The reordered head of a row is cut
// into chunks of 64 * UPL units (8 channels, one packed dword each); worker
// wave w quantizes chunk w % (NC + 1) (chunk NC: the outlier tail and the
// row's pitch padding) of row w / (NC + 1). It loads its permutation entries,
// then gathers the fp16 sources straight from global memory (a near-identity
// permutation reads whole cache lines, served from L1 after the first of the
// eight loads). An aligned
// segment of group / 8 lanes (one unit index i) is one group, so the group
// absmax is a few xor-shuffles. Codes and scales: the same arithmetic as the
// row kernel above (exact quotient, rint, offset nibbles).
template <int UPL, int TW>
__global__ __launch_bounds__(256) void quant_group_kernel(QuantArgs a, int NC) {
    const int lane = threadIdx.x & 63;
    const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
    const int c = gw % (NC + 1), row = gw / (NC + 1);
    if (row >= a.rows)
        return;
    const int K = a.K, K_n = a.K_n, G = a.G;
    const int U = (K_n + 7) / 8;
    const int W4 = (int)(a.pitch4 / 4), W8 = (int)(a.pitch8 / 4);
    const int seg = a.group / 8;                   // units per group: 16, 32, 64 or 64 UPL
    // entries are clamped into [0, K) once here, so that even a malformed
    // permutation (undefined behaviour by contract) reads inside the row
    auto pack = [K](int lo, int hi) {
        lo = min(max(lo, 0), K - 1);
        hi = min(max(hi, 0), K - 1);
        return (uint32_t)lo | ((uint32_t)hi << 16);
    };
    auto entry = [&](int j) { return a.perm ? a.perm[j] : j; };   // null: the identity order

    if (c < NC) {
        // ---- head chunk: units u = c * 64 UPL + 64 i + lane
        uint32_t pv[UPL][4];
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int u = c * 64 * UPL + 64 * i + lane, j0 = 8 * u;
            if (j0 + 8 <= K_n) {
                const int4 e0 = a.perm ? *reinterpret_cast<const int4 *>(a.perm + j0) : int4{j0, j0 + 1, j0 + 2, j0 + 3};
                const int4 e1 = a.perm ? *reinterpret_cast<const int4 *>(a.perm + j0 + 4)
                                       : int4{j0 + 4, j0 + 5, j0 + 6, j0 + 7};
                pv[i][0] = pack(e0.x, e0.y);
                pv[i][1] = pack(e0.z, e0.w);
                pv[i][2] = pack(e1.x, e1.y);
                pv[i][3] = pack(e1.z, e1.w);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    pv[i][k] = pack(j0 + 2 * k < K_n ? entry(j0 + 2 * k) : 0,
                                    j0 + 2 * k + 1 < K_n ? entry(j0 + 2 * k + 1) : 0);
            }
        }
        uint32_t v[UPL][4];
        {
            const uint16_t *src = reinterpret_cast<const uint16_t *>(a.src + (int64_t)row * a.ld);
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int j0 = 8 * (c * 64 * UPL + 64 * i + lane);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = j0 + 2 * k < K_n ? src[pv[i][k] & 0xFFFF] : 0u;
                    const uint32_t hi = j0 + 2 * k + 1 < K_n ? src[pv[i][k] >> 16] : 0u;
                    v[i][k] = lo | (hi << 16);
                }
            }
        }
        {
            uint32_t *q4row = reinterpret_cast<uint32_t *>(a.q4 + (int64_t)row * a.pitch4);
            // group absmax: over seg lanes of one unit index, and over all
            // of the chunk's units when a group is the whole chunk
            float gm[UPL];
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                half2 m2 = {(_Float16)0, (_Float16)0};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(half2, v[i][k] & 0x7FFF7FFFu));
                float m = fmaxf((float)m2.x, (float)m2.y);
                for (int off = 1; off < seg && off < 64; off <<= 1)
                    m = fmaxf(m, __shfl_xor(m, off, 64));
                gm[i] = m;
            }
            if (seg > 64) {
                float m = gm[0];
#pragma unroll
                for (int i = 1; i < UPL; ++i)
                    m = fmaxf(m, gm[i]);
#pragma unroll
                for (int i = 0; i < UPL; ++i)
                    gm[i] = m;
            }
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int u = c * 64 * UPL + 64 * i + lane;
                const float sc = gm[i] / 7.0f, rc = recip_or_zero(sc);
                if (u < U) {
                    if ((u & (seg - 1)) == 0)             // the group's first unit stores its scale
                        a.s4[(int64_t)row * G + (8 * u) / a.group] = sc;
                    uint32_t ev = 0, od = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float c0 = __builtin_rintf(exact_quotient((float)lo_half(v[i][k]), sc, rc)) + 8.0f;
                        const float c1 = __builtin_rintf(exact_quotient((float)hi_half(v[i][k]), sc, rc)) + 8.0f;
                        ev = __builtin_amdgcn_cvt_pk_u8_f32(c0, k, ev);
                        od = __builtin_amdgcn_cvt_pk_u8_f32(c1, k, od);
                    }
                    q4row[u] = (ev | (od << 4)) ^ 0x88888888u;
                }
            }
        }
        return;
    }

    // ---- the outlier tail (per-row INT8 scale) and the pitch padding of q4
    uint32_t pt[TW][2];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int j0 = K_n + 4 * (64 * i + lane);
#pragma unroll
        for (int k = 0; k < 2; ++k)
            pt[i][k] = pack(j0 + 2 * k < K ? entry(j0 + 2 * k) : 0, j0 + 2 * k + 1 < K ? entry(j0 + 2 * k + 1) : 0);
    }
    uint32_t tv[TW][2];
    {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(a.src + (int64_t)row * a.ld);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int j0 = K_n + 4 * (64 * i + lane);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t lo = j0 + 2 * k < K ? src[pt[i][k] & 0xFFFF] : 0u;
                const uint32_t hi = j0 + 2 * k + 1 < K ? src[pt[i][k] >> 16] : 0u;
                tv[i][k] = lo | (hi << 16);
            }
        }
    }
    {
        float tmax = 0.0f;
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const half2 h = __builtin_bit_cast(half2, tv[i][k] & 0x7FFF7FFFu);
                tmax = fmaxf(tmax, fmaxf((float)h.x, (float)h.y));
            }
        tmax = wave_max(tmax);
        const float s8 = tmax / 127.0f, r8 = recip_or_zero(s8);
        if (lane == 0 && a.s8)
            a.s8[row] = a.n_out > 0 ? s8 : 0.0f;
        if (a.q8) {
            uint32_t *q8row = reinterpret_cast<uint32_t *>(a.q8 + (int64_t)row * a.pitch8);
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                const int w = 64 * i + lane;
                if (w < W8) {
                    uint32_t word = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int j = K_n + 4 * w + k;
                        if (j < K) {
                            const uint32_t h = (k & 1) ? (tv[i][k >> 1] >> 16) : (tv[i][k >> 1] & 0xFFFF);
                            const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
                            const int q = (int)__builtin_rintf(exact_quotient(x, s8, r8));
                            word |= (uint32_t)(q & 0xFF) << (8 * k);
                        }
                    }
                    q8row[w] = word;
                }
            }
        }
        uint32_t *q4row = reinterpret_cast<uint32_t *>(a.q4 + (int64_t)row * a.pitch4);
        for (int u = U + lane; u < W4; u += 64)      // zero padding of the row pitch
            q4row[u] = 0u;
    }
}

// u6 producer with one 32-channel chunk per lane (per-row scales, or group
// scales of 128 channels; K a multiple of 8).
//
// The row kernel's u6 form spends most of its time on VALU work: about a dozen
// instructions per element for the quotient, the byte packing and the E2M3
// table lookups. Here each lane owns one whole chunk of the u6 operand (head
// channels 32c .. 32c + 31), so that gfx950's 32-value FP6 conversion
// (v_cvt_scalef32_pk32_fp6_f16) forms the chunk's 192-bit image in one
// instruction: with the integer codes q as fp16 inputs and a conversion scale
// of 8 it writes the E2M3 code of q / 8 of value i at bits 6i (every such
// quotient is exact in E2M3; the GPU tests check every code against the
// oracle's). Per element what remains is the exact
// quotient (three mixed-precision FMAs), rint and half a conversion to fp16.
// * Rows go global -> LDS by DMA in 16-byte pieces, with piece p stored in
//   slot p ^ ((p >> 4) & 15): a lane gathers the 32 channels of its chunk,
//   and without the swizzle the 64 lanes of a wave (chunks 64 bytes apart)
//   would meet in 4 of the 16 bank quads on every 2-byte read.
// * The LDS byte offsets of a lane's channels are the same for every row and
//   are formed once per workgroup (channels past the head, or past the tail,
//   point at 16 zero bytes after the row, so ragged chunks need no masks).
// * Two row buffers, refilled two rows ahead: once a row is gathered into
//   registers (second barrier) its buffer takes the row after next, so two
//   rows are in flight while one is coded.
// * Every store of a row is issued after the next row's wait and before the
//   DMA of the row after it, so the only memory operations younger than an
//   awaited row's DMA are one row's stores and the DMA behind it: the wait
//   is vmcnt(rounds) (never for the row in flight behind), and vmcnt(0) for
//   a workgroup's last row, which has no DMA behind it.
// * The tail words and the per-row scale stores go to the last lanes, whose
//   waves hold few or no head chunks.
// * Group scales (128 channels = 4 chunks = one aligned quad of lanes) need
//   two DPP steps; the per-row and tail maxima are reduced by DPP inside a
//   wave and through LDS across waves.
// * Codes are the definition's: q = rint(fl32(x / s)) by the exact quotient
//   (Markstein's correction from r = fl32(1 / s), exact for every fp16 x),
//   and the sign of a zero code is cleared before the conversion (E2M3 has a
//   negative zero; the operand's zero code is +0).
//
// Register budget: 80 VGPRs (six waves per SIMD) for the short-row buckets,
// which run several workgroups per CU; the 768-lane bucket runs one
// workgroup per CU (two 48 KB buffers).
template <int KMAX, int THREADS, bool GROUPED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(THREADS >= 768 ? 3 : 6)))
void quant_u6_chunk_kernel(QuantArgs a) {
    typedef _Float16 half32 __attribute__((ext_vector_type(32)));
    typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
    constexpr int NW = THREADS / 64;
    constexpr int ROUND = THREADS * 16;
    constexpr int XB = (KMAX * 2 + ROUND - 1) / ROUND * ROUND;
    constexpr int BUF = XB + 16;                   // row slots, then 16 zero bytes
    static_assert(THREADS * 32 >= KMAX, "one chunk per lane");
    static_assert(BUF < 65536, "offsets within a buffer fit 16 bits");
    __shared__ __align__(16) unsigned char xrow[2 * BUF];
    __shared__ uint32_t red_h[NW], red_t[NW];   // fp16 bits of the wave maxima

    const int K = a.K, K_n = a.K_n, n_out = a.n_out;
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nfull = K / 8;                       // 16-byte pieces of a row
    // the swizzle moves pieces within aligned runs of 16 slots: the DMA covers
    // every slot up to the end of the last run
    const int rounds = (((nfull + 15) & ~15) + THREADS - 1) / THREADS;
    const int NCH = (int)(a.pitch4 / 16);          // chunks of the padded head
    const int W8 = (int)(a.pitch8 / 4);
    const int64_t T6 = a.pitch4 / 32;
    // tail words go to the last W8 lanes (whose waves hold fewer head
    // chunks), and so do the per-row scale stores
    const int tw = tid - (THREADS - W8);

    auto issue_row = [&](int row, int b) {
        const unsigned char *src = reinterpret_cast<const unsigned char *>(a.src + (int64_t)row * a.ld);
        const uint32_t d = lds_addr(xrow + b * BUF) + wave_u * 1024;
        for (int j = 0; j < rounds; ++j) {
            const int slot = j * THREADS + tid;
            const int piece = slot ^ ((slot >> 4) & 15);
            dma16_stream(src, (uint32_t)(piece < nfull ? piece : 0) * 16, d + j * ROUND);
        }
    };
    int row = blockIdx.x;
    if (gridDim.x % 8 == 0)                        // consecutive rows on one XCD (see the row kernel)
        row = (int)((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8);
    if (row < a.rows)
        issue_row(row, 0);
    if (row + (int)gridDim.x < a.rows)
        issue_row(row + gridDim.x, 1);
    if (tid < 8)
        reinterpret_cast<uint32_t *>(xrow + (tid >> 2) * BUF + XB)[tid & 3] = 0u;

    // LDS byte offsets (within a buffer) of the lane's 32 head channels and 4
    // tail channels, two per register. The permutation entries are all
    // requested before any is used: head entries as 16-byte loads (K is a
    // multiple of 8, so K / 4 whole int4s), tail entries one by one, indices
    // clamped into the array and entries into the row.
    auto slot_of = [&](int ch) -> uint32_t {
        ch = min(max(ch, 0), K - 1);
        const int piece = ch >> 3;
        return (uint32_t)((piece ^ ((piece >> 4) & 15)) * 16 + (ch & 7) * 2);
    };
    // (kept unpacked where one workgroup per CU leaves registers to spare)
    constexpr bool PACKED = THREADS < 768;
    uint32_t off[16], toff[2], offu[PACKED ? 1 : 32], toffu[PACKED ? 1 : 4];
    {
        int e[32], t[4];
        if (a.perm) {
            const int4 *perm4 = reinterpret_cast<const int4 *>(a.perm);
            const int last4 = K / 4 - 1;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int4 q = perm4[min(8 * tid + m, last4)];
                e[4 * m] = q.x;
                e[4 * m + 1] = q.y;
                e[4 * m + 2] = q.z;
                e[4 * m + 3] = q.w;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                t[k] = a.perm[min(K_n + 4 * max(tw, 0) + k, K - 1)];
        } else {
#pragma unroll
            for (int k = 0; k < 32; ++k)
                e[k] = 32 * tid + k;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                t[k] = K_n + 4 * tw + k;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int j = 32 * tid + 2 * k;
            off[k] = (j < K_n ? slot_of(e[2 * k]) : (uint32_t)XB) |
                     ((j + 1 < K_n ? slot_of(e[2 * k + 1]) : (uint32_t)XB) << 16);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int j = K_n + 4 * tw + 2 * k;
            toff[k] = ((tw >= 0 && j < K) ? slot_of(t[2 * k]) : (uint32_t)XB) |
                      (((tw >= 0 && j + 1 < K) ? slot_of(t[2 * k + 1]) : (uint32_t)XB) << 16);
        }
        if constexpr (!PACKED) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                offu[2 * k] = off[k] & 0xFFFF;
                offu[2 * k + 1] = off[k] >> 16;
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                toffu[2 * k] = toff[k] & 0xFFFF;
                toffu[2 * k + 1] = toff[k] >> 16;
            }
        }
    }
    // the lane's places in a row block: image bytes 0..15 and 16..23 of its chunk
    const uint32_t lo_off = (uint32_t)(tid >> 1) * (uint32_t)kU6Block + 512u * (uint32_t)(tid & 1);
    const uint32_t hi_off = (uint32_t)(tid >> 1) * (uint32_t)kU6Block + 1024u + 256u * (uint32_t)(tid & 1);

    // the previous row's results, stored after the next wait
    int prow = -1;
    u32x6 img = {0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t word = 0;
    float psc = 0.0f, ps8 = 0.0f;
    auto store_prev = [&]() {
        if (prow < 0)
            return;
        if (tid < NCH) {
            // uniform row-block base + the lane's own 32-bit offsets (the
            // stores then need no 64-bit lane pointers)
            unsigned char *rowblk = a.u6 + (int64_t)(prow >> 5) * T6 * kU6Block;
            const int rr = prow & 31;
            *reinterpret_cast<uint4 *>(rowblk + 16 * rr + lo_off) = uint4{img[0], img[1], img[2], img[3]};
            *reinterpret_cast<uint2 *>(rowblk + 8 * rr + hi_off) = uint2{img[4], img[5]};
        }
        if (GROUPED) {
            if (tid < NCH && (tid & 3) == 0 && 32 * tid < K_n)
                a.s4[(int64_t)prow * a.G + (tid >> 2)] = psc;
        } else if (tid == THREADS - 1 && a.G > 0) {
            a.s4[prow] = psc;
        }
        if (tid == THREADS - 1 && a.s8)
            a.s8[prow] = n_out > 0 ? ps8 : 0.0f;
        if (tw >= 0 && a.q8) {
            uint32_t o8 = 4u * (uint32_t)tw;   // (kept apart from the base: no 64-bit lane pointer)
            asm volatile("" : "+v"(o8));
            *reinterpret_cast<uint32_t *>(a.q8 + (int64_t)prow * a.pitch8 + o8) = word;
        }
    };

    // one row from buffer B (a constant, so that the buffer base is the LDS
    // reads' immediate offset)
    auto do_row = [&](auto b_tag) {
        constexpr int B = decltype(b_tag)::value;
        // (1) this row's DMA has landed in every wave, and this wave's LDS
        //     writes are done (lgkmcnt(0)). Younger than the DMA are the
        //     previous row's stores and, unless this is the workgroup's last
        //     row, the next row's DMA: vmcnt(rounds) then (all but the
        //     youngest DMA's instructions), vmcnt(0) otherwise.
        asm volatile("" ::: "memory");
        if (row + (int)gridDim.x < a.rows) {
            switch (rounds) {                      // s_waitcnt takes an immediate: vmcnt(n) lgkmcnt(0)
                case 1: __builtin_amdgcn_s_waitcnt(0x071); break;
                case 2: __builtin_amdgcn_s_waitcnt(0x072); break;
                case 3: __builtin_amdgcn_s_waitcnt(0x073); break;
                case 4: __builtin_amdgcn_s_waitcnt(0x074); break;
                default: __builtin_amdgcn_s_waitcnt(kWaitAll); break;
            }
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitAll);
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        store_prev();

        // (2) gather the chunk and the tail word; maxima (the offsets are
        //     unpacked here, not kept unpacked across the loop)
        const unsigned char *xb = xrow + B * BUF;
        half2 v[16], tv[2];
        if constexpr (PACKED) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                asm volatile("" : "+v"(off[k]));
#pragma unroll
            for (int k = 0; k < 2; ++k)
                asm volatile("" : "+v"(toff[k]));
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                v[p].x = *reinterpret_cast<const _Float16 *>(xb + (off[p] & 0xFFFF));
                v[p].y = *reinterpret_cast<const _Float16 *>(xb + (off[p] >> 16));
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                tv[p].x = *reinterpret_cast<const _Float16 *>(xb + (toff[p] & 0xFFFF));
                tv[p].y = *reinterpret_cast<const _Float16 *>(xb + (toff[p] >> 16));
            }
        } else {
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                v[p].x = *reinterpret_cast<const _Float16 *>(xb + offu[2 * p]);
                v[p].y = *reinterpret_cast<const _Float16 *>(xb + offu[2 * p + 1]);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                tv[p].x = *reinterpret_cast<const _Float16 *>(xb + toffu[2 * p]);
                tv[p].y = *reinterpret_cast<const _Float16 *>(xb + toffu[2 * p + 1]);
            }
        }
        // |x| as fp16 bits: non-negative values order like unsigned integers
        typedef uint16_t ushort2_t __attribute__((ext_vector_type(2)));
        const ushort2_t mag = {0x7FFF, 0x7FFF};
        ushort2_t m2 = __builtin_bit_cast(ushort2_t, v[0]) & mag;
#pragma unroll
        for (int p = 1; p < 16; ++p)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(ushort2_t, v[p]) & mag);
        const ushort2_t t2 = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, tv[0]) & mag,
                                                       __builtin_bit_cast(ushort2_t, tv[1]) & mag);
        // (fp16 bits of |x| widen to an order-preserving integer: the maxima
        // are taken on the bits and converted once)
        uint32_t hm = __builtin_elementwise_max(m2.x, m2.y);
        hm = dpp_max_u32<0xB1>(hm);               // quad: lanes ^ 1
        hm = dpp_max_u32<0x4E>(hm);               // quad: lanes ^ 2 (one 128-channel group)
        if (!GROUPED)
            hm = wave_max_of_quads(hm);
        const bool tail_wave = (int)wave_u * 64 + 64 > THREADS - W8;   // uniform: the wave holds tail words
        uint32_t tm = 0;
        if (tail_wave)
            tm = wave_max_dpp(__builtin_elementwise_max(t2.x, t2.y));
        if (lane == 0) {
            if (!GROUPED)
                red_h[wave_u] = hm;
            red_t[wave_u] = tm;
        }
        // (3) every wave has its values: the buffer takes the row after next
        lds_barrier();
        if (row + 2 * (int)gridDim.x < a.rows)
            issue_row(row + 2 * gridDim.x, B);

        uint32_t rb = hm, tb = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if (!GROUPED)
                rb = max(rb, red_h[w]);
            tb = max(tb, red_t[w]);
        }
        const float ra = (float)__builtin_bit_cast(_Float16, (uint16_t)rb);
        const float ta = (float)__builtin_bit_cast(_Float16, (uint16_t)tb);
        const float sc = div_small_const(ra, 7.0f, 1.0f / 7.0f), rc = recip_or_zero(sc);
        const float s8 = div_small_const(ta, 127.0f, 1.0f / 127.0f);

        // (4) head codes -> E2M3 image of the chunk (waves wholly past the
        //     head skip it; other lanes past it hold zeros, never stored)
        if ((int)wave_u * 64 < NCH) {
            half32 q;
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const float c0 = __builtin_rintf(exact_quotient_h(v[p].x, sc, rc));
                const float c1 = __builtin_rintf(exact_quotient_h(v[p].y, sc, rc));
                const half2 h = __builtin_bit_cast(half2, __builtin_amdgcn_cvt_pkrtz(c0, c1)) + (half2){0, 0};
                q[2 * p] = h.x;
                q[2 * p + 1] = h.y;
            }
            img = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(q, 8.0f);
        }
        // (5) INT8 tail word (waves that hold tail words)
        if (tail_wave) {
            const float r8 = recip_or_zero(s8);
            word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const _Float16 x = (k & 1) ? tv[k >> 1].y : tv[k >> 1].x;
                const int qi = (int)__builtin_rintf(exact_quotient_h(x, s8, r8));
                word |= (uint32_t)(qi & 0xFF) << (8 * k);
            }
        }
        psc = sc;
        ps8 = s8;
        prow = row;
        row += gridDim.x;
    };
    while (row < a.rows) {
        do_row(std::integral_constant<int, 0>{});
        if (row >= a.rows)
            break;
        do_row(std::integral_constant<int, 1>{});
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    store_prev();

    // rows past the last one, up to the end of its 32-row block: code 0
    const int rows_padded = (a.rows + 31) & ~31;
    for (int zr = a.rows + (int)blockIdx.x; zr < rows_padded; zr += (int)gridDim.x)
        if (tid < NCH) {
            unsigned char *rowblk = a.u6 + (int64_t)(zr >> 5) * T6 * kU6Block;
            const int rr = zr & 31;
            *reinterpret_cast<uint4 *>(rowblk + 16 * rr + lo_off) = uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint2 *>(rowblk + 8 * rr + hi_off) = uint2{0u, 0u};
        }
}

// Resident workgroups of one instantiation on the current device, queried on
// first use (a launch then costs no runtime queries).
template <int KMAX, int THREADS, bool GROUPED, bool WIDE_TAIL, bool NORM, bool FULL, bool U6>
long resident_slots() {
    static std::atomic<long> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        dev = -1;
    if (dev >= 0) {
        const long c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 256, per_cu = 1;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_kernel<KMAX, THREADS, GROUPED, WIDE_TAIL, NORM, FULL, U6>,
                                                     THREADS, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long slots = (long)cus * per_cu;
    if (dev >= 0)
        cached[dev].store(slots, std::memory_order_relaxed);
    return slots;
}

template <int KMAX, int THREADS, bool GROUPED>
long u6_chunk_slots() {
    static std::atomic<long> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        dev = -1;
    if (dev >= 0) {
        const long c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 256, per_cu = 1;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_u6_chunk_kernel<KMAX, THREADS, GROUPED>, THREADS, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const long slots = (long)cus * per_cu;
    if (dev >= 0)
        cached[dev].store(slots, std::memory_order_relaxed);
    return slots;
}

template <int KMAX, int THREADS, bool GROUPED>
hipError_t launch_u6_chunk_bucket(const QuantArgs &a, hipStream_t stream) {
    const int grid = (int)std::min<long>(a.rows, u6_chunk_slots<KMAX, THREADS, GROUPED>());
    hipLaunchKernelGGL((quant_u6_chunk_kernel<KMAX, THREADS, GROUPED>), dim3(grid), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

// The chunk kernel takes K a multiple of 8, per-row or 128-channel group
// scales and a tail of at most one 4-channel word per lane; false: use the
// row kernel.
template <bool GROUPED>
bool launch_u6_chunk(const QuantArgs &a, hipStream_t stream, hipError_t *err) {
    if (a.K % 8 != 0 || (GROUPED && a.group != 128))
        return false;
    const int64_t words = a.pitch8 / 4;
    if (a.K <= 4096 && words <= 128) *err = launch_u6_chunk_bucket<4096, 128, GROUPED>(a, stream);
    else if (a.K <= 8192 && words <= 256) *err = launch_u6_chunk_bucket<8192, 256, GROUPED>(a, stream);
    else if (a.K <= 16384 && words <= 512) *err = launch_u6_chunk_bucket<16384, 512, GROUPED>(a, stream);
    else if (a.K <= 24576 && words <= 768) *err = launch_u6_chunk_bucket<24576, 768, GROUPED>(a, stream);
    else return false;
    return true;
}

template <int KMAX, int THREADS, bool GROUPED, bool WIDE_TAIL, bool NORM, bool FULL, bool U6>
hipError_t launch_tail(const QuantArgs &a, hipStream_t stream) {
    const int grid = (int)std::min<long>(a.rows, resident_slots<KMAX, THREADS, GROUPED, WIDE_TAIL, NORM, FULL, U6>());
    hipLaunchKernelGGL((quant_rows_kernel<KMAX, THREADS, GROUPED, WIDE_TAIL, NORM, FULL, U6>), dim3(grid),
                       dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

template <int KMAX, int THREADS, bool GROUPED, bool NORM, bool U6>
hipError_t launch(const QuantArgs &a, hipStream_t stream) {
    if (a.pitch8 / 4 > THREADS)                   // more than one tail word per lane
        return launch_tail<KMAX, THREADS, GROUPED, true, NORM, false, U6>(a, stream);
    if (a.K % 8 == 0 && a.K_n % 8 == 0)           // every unit and tail word inside the row
        return launch_tail<KMAX, THREADS, GROUPED, false, NORM, true, U6>(a, stream);
    return launch_tail<KMAX, THREADS, GROUPED, false, NORM, false, U6>(a, stream);
}

// Row-length buckets: (longest row, lanes per workgroup).
template <bool GROUPED, bool NORM, bool U6 = false>
hipError_t launch_grouping(const QuantArgs &a, hipStream_t stream) {
    if (a.K <= 4096) return launch<4096, 256, GROUPED, NORM, U6>(a, stream);
    if (a.K <= 8192) return launch<8192, 512, GROUPED, NORM, U6>(a, stream);
    if (a.K <= 16384) return launch<16384, 1024, GROUPED, NORM, U6>(a, stream);
    if (a.K <= 24576) return launch<24576, 1024, GROUPED, NORM, U6>(a, stream);
    return hipErrorInvalidValue;
}

// The group kernel serves short batches (decode): one worker wave per
// (row, chunk), so a row's chunks are quantized side by side. Longer batches
// keep the row kernel, which measured faster there (its row DMA keeps more
// bytes in flight per instruction than eight 2-byte gathers).
constexpr int kGroupUPL = 2;
constexpr int kGroupMaxRows = 64;

template <int TW>
hipError_t launch_group(const QuantArgs &a, hipStream_t stream) {
    const int U = (a.K_n + 7) / 8;
    const int NC = (U + 64 * kGroupUPL - 1) / (64 * kGroupUPL);
    const long waves = (long)(NC + 1) * a.rows;
    const int grid = (int)((waves + 3) / 4);
    hipLaunchKernelGGL((quant_group_kernel<kGroupUPL, TW>), dim3(grid), dim3(256), 0, stream, a, NC);
    return hipGetLastError();
}

}  // namespace quant_impl

int quant_rows_max_k() { return 24576; }

hipError_t launch_quant_rows(const QuantArgs &a, hipStream_t stream) {
    if (a.rows == 0)
        return hipSuccess;
    if (a.u6) {                                   // u6 head: chunk kernel, else (and with the norm) the row kernel
        if (a.gamma)
            return a.group > 0 ? quant_impl::launch_grouping<true, true, true>(a, stream)
                               : quant_impl::launch_grouping<false, true, true>(a, stream);
        hipError_t err = hipSuccess;
        if (a.group > 0 ? quant_impl::launch_u6_chunk<true>(a, stream, &err)
                        : quant_impl::launch_u6_chunk<false>(a, stream, &err))
            return err;
        return a.group > 0 ? quant_impl::launch_grouping<true, false, true>(a, stream)
                           : quant_impl::launch_grouping<false, false, true>(a, stream);
    }
    if (a.gamma)                                  // the norm needs whole rows: row kernel
        return a.group > 0 ? quant_impl::launch_grouping<true, true>(a, stream)
                           : quant_impl::launch_grouping<false, true>(a, stream);
    if (a.rows <= quant_impl::kGroupMaxRows &&
        (a.group == 128 || a.group == 256 || a.group == 512 || a.group == 64 * 8 * quant_impl::kGroupUPL)) {
        const int tw = (int)((a.pitch8 / 4 + 63) / 64);
        if (tw <= 1) return quant_impl::launch_group<1>(a, stream);
        if (tw <= 2) return quant_impl::launch_group<2>(a, stream);
        if (tw <= 4) return quant_impl::launch_group<4>(a, stream);
    }
    return a.group > 0 ? quant_impl::launch_grouping<true, false>(a, stream)
                       : quant_impl::launch_grouping<false, false>(a, stream);
}

}  // namespace w4a4
