// Decode layer call with the activation quantizer fused into the GEMM: for
// batches of at most 2 token rows with 128-channel groups, the fp16 tokens are
// gathered, quantized and packed inside the GEMM workgroups, so the layer is
// one launch and the codes never travel through memory.
//
// Method: Atom summary page (Summary paragraph 2: activation scales computed
// for every input at run time, INT4 groups plus an 8-bit outlier part over
// reordered channels; Interesting ideas I2: the reordering and quantization
// fused into the operators next to the GEMM) and the QUIK abstract (one-token
// decode is memory-bound, so the weights set the time).
//
// CDNA4 design (HBM-bound on the weights, which are read once)
// * The column stripes, K ranges, weight DMA and fold are those of the decode
//   GEMM: a workgroup owns 32 output columns, its eight waves split the INT4
//   K-tiles into contiguous ranges, each wave streams pairs of weight tiles
//   into an LDS ring of its own, and each tile is folded at once with a
//   v_mfma_f32_32x32x2f32 scale product. (A four-slot ring, eight tiles of a
//   wave in flight during the quantizer, measured slower than two slots.)
// * With 128-channel groups a K-tile is one scale group, so a wave needs the
//   token codes and scales of its own tiles only: no workgroup barrier stands
//   between the quantizer and the MFMAs. A lane takes unit columns of 8
//   reordered channels (one packed dword of codes): it loads their 8
//   permutation entries once and gathers the fp16 values of every token row;
//   an aligned 16-lane segment is one group, so its absmax is four
//   xor-shuffles. Codes use the row quantizer's arithmetic (s = absmax / 7,
//   r = 1 / s, the exact quotient by Markstein's correction, rint), so they
//   are bit-identical to the producer's and the result equals the two-launch
//   path bit for bit.
// * The codes go to a wave-private LDS area in the token layout of the pair
//   slots (row stride padded so that the rows of one read fall on distinct
//   banks); the group scales beside them.
// * The INT8 tail (at most 128 channels, one tile per wave 0 and 1): a tail
//   wave gathers all tail channels of every token row for the row's absmax,
//   then codes the 64 channels of its own tile into LDS.
// * With the RMSNorm in front (NORM): each wave adds the squares of its own
//   channels exactly, as 128-bit integers of x^2 * 2^48 (wave 0 also the
//   tail's), the eight partial sums meet in LDS behind one barrier, and every
//   lane derives rstd = fl32(1 / sqrt(fl64(S) / K + eps)) in binary64 and
//   normalizes its values as fl16(gamma * fl16(fl32(x * rstd))) before the
//   absmax: the producer's arithmetic, so the codes stay bit-identical.
// * Loads complete in order, so the waits are counted by hand around the
//   weight DMA: the first two pairs are requested before the permutation
//   entries arrive (their HBM latency overlaps the quantizer); with a deeper
//   ring, further pairs would follow the token gathers and stay in flight
//   while the codes are computed.
#include "gemm_common.h"

namespace w4a4 {
namespace decode_fused_impl {

using namespace gemm_impl;

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int WAVES = 8, THREADS = WAVES * 64;
constexpr int BN = 32;                     // output columns per workgroup
constexpr int MAXM = 2;                    // token rows (each costs every workgroup its codes)
constexpr int MAXT = 16;                   // INT4 tiles per wave (K_n <= 16384)
constexpr int UCW = MAXT * 16 / 64;        // unit columns per lane
constexpr int MAXOUT = 128;                // outlier channels (two tail tiles)
constexpr int PAIR = 128;                  // bytes of a weight row in a pair of tiles
constexpr int WSLOT = 32 * PAIR;           // 32 weight rows
constexpr int SLOTS = 2;                   // weight pairs in flight per wave
constexpr int RING = WAVES * SLOTS * WSLOT;
constexpr int TROW = MAXT * kTileBytes + 32;   // token row stride: rows 32 bytes apart modulo 256
constexpr int TOK = MAXM * TROW;           // INT4 token codes of one wave
constexpr int TAIL = MAXM * kTileBytes;    // INT8 codes of the wave's tail tile
constexpr int SCL = MAXM * MAXT * 4 + MAXM * 4;   // group scales, then tail scales
constexpr int WAVE_AREA = TOK + TAIL + SCL;
constexpr int SUMS = WAVES * MAXM * 16;      // partial sums of squares (RMSNorm), 128 bits each
constexpr int WSC = 32 * MAXT * 4;         // weight scales of a wave's tiles, [32 rows][nt]
constexpr int LDS_BYTES = RING + WAVES * WAVE_AREA + SUMS + WAVES * WSC;
constexpr int RED_BYTES = WAVES * 16 * 64 * 4;
static_assert(RING >= RED_BYTES, "the reduction reuses the ring");
static_assert(LDS_BYTES <= 160 * 1024, "one workgroup per CU");

__device__ __forceinline__ v4i as_v4i(uint4 p) { return v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w}; }

// 16-byte chunk c of row r of a pair slot sits at chunk position c ^ (r & 7)
__device__ __forceinline__ int pair_off(int r, int c) { return r * PAIR + ((c ^ (r & 7)) << 4); }

// fl32(x / s) from r = fl32(1 / s); r == 0 encodes s == 0 (then x == 0 too).
__device__ __forceinline__ float exact_quotient(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, r, q0);
}

__device__ __forceinline__ float recip_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// x^2 * 2^48 of an fp16 value, exactly, as an integer below 2^80: with
// x = Mx * 2^(sh - 24) (Mx the significand with its hidden bit, sh = 0 for
// subnormals), x^2 * 2^48 = Mx^2 * 2^(2 sh).
__device__ __forceinline__ unsigned __int128 square_q48(uint16_t h) {
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

// fl16(gamma * fl16(fl32(x * rstd))): the fp16 product of two fp16 values is
// exact in fp32, so one rounding to fp16 gives the fp16 multiply.
__device__ __forceinline__ uint16_t norm_one(uint16_t x, uint16_t g, float rstd) {
#pragma clang fp contract(off)
    const _Float16 h = (_Float16)(h2f(x) * rstd);
    return __builtin_bit_cast(uint16_t, (_Float16)((float)h * h2f(g)));
}

template <bool NORM>
__global__ __launch_bounds__(THREADS) void decode_fused_kernel(DecodeFusedArgs a) {
    __shared__ __align__(16) unsigned char lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    const int n0 = blockIdx.x * BN;
    const int T4 = a.K_n / 128, T8 = (a.n_out + 63) / 64, G = T4;
    const int per = (T4 + WAVES - 1) / WAVES;                 // <= MAXT (checked at launch)
    const int tb = min(wave * per, T4), te = min(tb + per, T4);
    const int nt = te - tb, np = (nt + 1) / 2;                // tiles and pairs of this wave

    unsigned char *wl = lds + wave * SLOTS * WSLOT;           // weight ring of this wave
    unsigned char *tok = lds + RING + wave * WAVE_AREA;       // [MAXM][TROW] INT4 codes
    unsigned char *tail = tok + TOK;                          // [MAXM][64] INT8 codes
    float *tsc = reinterpret_cast<float *>(tail + TAIL);      // [MAXM][MAXT] group scales
    float *t8s = tsc + MAXM * MAXT;                           // [MAXM] tail scales

    const int64_t nrow = min(n0 + li, a.N - 1);
    const int mrow = min(li, a.M - 1);
    const bool tail_wave = T8 > wave;

    // ---- loads that do not depend on anything: weight scales and tail ------------
    // The weight scales of the wave's tiles (32 rows x nt floats, nt
    // consecutive floats per row) go to LDS by DMA of 4 bytes per lane, a
    // row segment to consecutive lanes, so an instruction touches two to
    // eight rows instead of the 32 that a per-lane load of one tile's scale
    // touches. They are older than every later load, so the first wait on a
    // pair covers them.
    float *swl = reinterpret_cast<float *>(lds + RING + WAVES * WAVE_AREA + SUMS + wave * WSC);
    {
        const int units = 32 * nt, rmax = a.N - 1 - n0;
        const float *sbase = a.sw4 + (int64_t)n0 * G + tb;
        for (int i = 0; i * 64 < units; ++i) {
            const int u = min(i * 64 + lane, units - 1), r = u / nt, k = u - r * nt;
            dma4s(sbase, 4u * (uint32_t)(min(r, rmax) * G + k), lds_addr(swl) + i * 256);
        }
    }
    const int swr = (int)(nrow - n0) * nt;
    const uint8_t *w8row = reinterpret_cast<const uint8_t *>(a.w8) + nrow * a.pitch8 + 16 * lh;
    uint4 tw[2] = {};
    if (tail_wave) {
        tw[0] = *reinterpret_cast<const uint4 *>(w8row + wave * kTileBytes);
        tw[1] = *reinterpret_cast<const uint4 *>(w8row + wave * kTileBytes + 32);
    }

    // ---- permutation entries: unit column c = lane + 64 i holds reordered
    // channels tb * 128 + 8 c .. + 7 (live when c < nt * 16, uniform per 16-lane
    // segment); tail channel c = lane + 64 i of the outlier segment
    const uint32_t kmax = (uint32_t)(a.K - 1);
    const int ucols = nt * 16;                                // live unit columns of the wave
    int4 pe[UCW][2];
#pragma unroll
    for (int i = 0; i < UCW; ++i) {
        if (64 * i >= ucols)
            break;                                            // uniform
        const int c = lane + 64 * i;
        const int j0 = c < ucols ? tb * 128 + 8 * c : 0;      // clamped into the array
        pe[i][0] = *reinterpret_cast<const int4 *>(a.perm + j0);
        pe[i][1] = *reinterpret_cast<const int4 *>(a.perm + j0 + 4);
    }
    int pt[2] = {0, 0};
    if (tail_wave) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            pt[i] = a.perm[a.K_n + min(lane + 64 * i, a.n_out - 1)];
    }

    // ---- DMA of a pair of weight tiles: instruction i covers rows 8 i .. 8 i + 7,
    // lane q row 8 i + q / 8 and stored chunk q % 8 (logical chunk (q % 8) ^ (row & 7));
    // chunks 4..7 are the second tile, or the first again past the last tile
    uint32_t ow[4], owd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3), c = (lane & 7) ^ (r & 7);
        const int64_t wr = min(n0 + r, a.N - 1);
        ow[i] = (uint32_t)(wr * a.pitch4) + 16 * c;
        owd[i] = (uint32_t)(wr * a.pitch4) + 16 * (c & 3);
    }
    auto issue = [&](int j) {                                 // pair j into slot j % SLOTS
        const int t0 = tb + 2 * j;
        const bool dup = t0 + 1 >= te;                        // odd last pair: no second tile
        const uint32_t st = lds_addr(wl + (j % SLOTS) * WSLOT);
        const uint8_t *W = a.w4 + t0 * kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(W, dup ? owd[i] : ow[i], st + i * 1024);
    };
    // s_waitcnt leaving the DMA of `pairs` pairs (4 instructions each) outstanding
    auto wait_pairs = [&](int pairs) {
        switch (pairs) {
        case 0: __builtin_amdgcn_s_waitcnt(vmcnt_only(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vmcnt_only(4)); break;
        default: __builtin_amdgcn_s_waitcnt(vmcnt_only(8)); break;
        }
    };
    const int early = min(np, 2), late = min(np, SLOTS) - early;
    for (int j = 0; j < early; ++j)
        issue(j);

    // ---- token gathers, once the permutation entries (older than the DMA of
    // pairs 0 and 1) are back
    compiler_fence();
    wait_pairs(early);
    compiler_fence();
    const uint16_t *X = a.x;
    uint16_t xv[MAXM][UCW][8];
#pragma unroll
    for (int i = 0; i < UCW; ++i) {
        if (64 * i >= ucols)
            break;                                            // uniform
        const int p[8] = {pe[i][0].x, pe[i][0].y, pe[i][0].z, pe[i][0].w,
                          pe[i][1].x, pe[i][1].y, pe[i][1].z, pe[i][1].w};
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
            const uint16_t *row = X + (int64_t)r * a.ldx;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xv[r][i][e] = row[min((uint32_t)p[e], kmax)];
        }
    }
    uint16_t xt[MAXM][2] = {};
    if (tail_wave) {
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
#pragma unroll
            for (int i = 0; i < 2; ++i)
                xt[r][i] = X[(int64_t)r * a.ldx + min((uint32_t)pt[i], kmax)];
        }
    }
    uint16_t gv[UCW][8], gt[2] = {0, 0};                      // norm weights of the same channels
    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < UCW; ++i) {
            if (64 * i >= ucols)
                break;                                        // uniform
            const int p[8] = {pe[i][0].x, pe[i][0].y, pe[i][0].z, pe[i][0].w,
                              pe[i][1].x, pe[i][1].y, pe[i][1].z, pe[i][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                gv[i][e] = a.gamma[min((uint32_t)p[e], kmax)];
        }
        if (tail_wave) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                gt[i] = a.gamma[min((uint32_t)pt[i], kmax)];
        }
    }
    for (int j = early; j < early + late; ++j)
        issue(j);
    compiler_fence();
    wait_pairs(late);                                         // the token loads and every older load
    compiler_fence();

    if constexpr (NORM) {
        // exact sums of squares: this wave's head channels, and wave 0 adds the tail
        uint32_t *sums = reinterpret_cast<uint32_t *>(lds + RING + WAVES * WAVE_AREA);   // [WAVES][MAXM][4]
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
            unsigned __int128 ss = 0;
#pragma unroll
            for (int i = 0; i < UCW; ++i) {
                if (64 * i >= ucols)
                    break;                                    // uniform
                if (lane + 64 * i < ucols)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ss += square_q48(xv[r][i][e]);
            }
            if (wave == 0 && tail_wave)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if (lane + 64 * i < a.n_out)
                        ss += square_q48(xt[r][i]);
            ss = wave_sum_u128(ss);
            if (lane == 0)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    sums[(wave * MAXM + r) * 4 + k] = (uint32_t)(ss >> (32 * k));
        }
        // a barrier that orders LDS only: the weight DMA keeps running across it
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
            unsigned __int128 S = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint32_t *q = sums + (w * MAXM + r) * 4;
                S += (unsigned __int128)q[0] | ((unsigned __int128)q[1] << 32) | ((unsigned __int128)q[2] << 64) |
                     ((unsigned __int128)q[3] << 96);
            }
            const double var = (double)S * 0x1p-48 / (double)a.K + (double)a.eps;
            const float rstd = var == 0.0 ? 0.0f : (float)(1.0 / __builtin_sqrt(var));
#pragma unroll
            for (int i = 0; i < UCW; ++i) {
                if (64 * i >= ucols)
                    break;                                    // uniform
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xv[r][i][e] = norm_one(xv[r][i][e], gv[i][e], rstd);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                xt[r][i] = norm_one(xt[r][i], gt[i], rstd);
        }
    }

    // ---- INT4 codes and group scales of this wave's tiles ---------------------------
#pragma unroll
    for (int i = 0; i < UCW; ++i) {
        if (64 * i >= ucols)
            break;                                            // uniform
        const int c = lane + 64 * i;
        const bool live = c < ucols;                          // uniform per 16-lane segment
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
            float v[8], m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[e] = h2f(xv[r][i][e]);
                m = fmaxf(m, fabsf(v[e]));
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1)            // the group's 16 lanes
                m = fmaxf(m, __shfl_xor(m, off, 64));
            const float s = m / 7.0f, rc = recip_or_zero(s);
            uint32_t ev = 0, od = 0;                          // offset codes of even / odd channels
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(v[2 * k], s, rc)) + 8.0f, k, ev);
                od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(exact_quotient(v[2 * k + 1], s, rc)) + 8.0f, k, od);
            }
            if (live) {
                *reinterpret_cast<uint32_t *>(tok + r * TROW + 4 * c) = (ev | (od << 4)) ^ 0x88888888u;
                if ((c & 15) == 0)
                    tsc[r * MAXT + (c >> 4)] = s;
            }
        }
    }

    // ---- INT8 tail: row absmax over every outlier channel, codes of this wave's tile
    if (tail_wave) {
#pragma unroll
        for (int r = 0; r < MAXM; ++r) {
            if (r >= a.M)
                break;                                        // uniform
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (lane + 64 * i < a.n_out)
                    m = fmaxf(m, fabsf(h2f(xt[r][i])));
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                m = fmaxf(m, __shfl_xor(m, off, 64));
            const float s8 = m / 127.0f, r8 = recip_or_zero(s8);
            // channel 64 * wave + lane: this lane's own value (i = wave), zero past n_out
            const int c = 64 * wave + lane;
            const float x = c < a.n_out ? h2f(wave == 0 ? xt[r][0] : xt[r][1]) : 0.0f;
            const int q = (int)__builtin_rintf(exact_quotient(x, s8, r8));
            tail[r * kTileBytes + lane] = (uint8_t)(int8_t)q;
            if (lane == 0)
                t8s[r] = s8;
        }
    }
    // the wave reads back only what it wrote itself (LDS is in order per wave)
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    compiler_fence();

    float sa[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k)
        sa[k] = k < nt ? tsc[mrow * MAXT + k] : 0.0f;
    const unsigned char *trow = tok + mrow * TROW;

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
            const uint4 px = *reinterpret_cast<const uint4 *>(trow + k * kTileBytes + (2 * s + lh) * 16);
            const v4i w0 = {(int)nib_lo(pw.x), (int)nib_hi(pw.x), (int)nib_lo(pw.y), (int)nib_hi(pw.y)};
            const v4i w1 = {(int)nib_lo(pw.z), (int)nib_hi(pw.z), (int)nib_lo(pw.w), (int)nib_hi(pw.w)};
            const v4i x0 = {(int)nib_lo(px.x), (int)nib_hi(px.x), (int)nib_lo(px.y), (int)nib_hi(px.y)};
            const v4i x1 = {(int)nib_lo(px.z), (int)nib_hi(px.z), (int)nib_lo(px.w), (int)nib_hi(px.w)};
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0, x0, s == 0 ? zi : acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1, x1, acc, 0, 0, 0);
        }
        // scale products S[n][m] = sw[n] * sa[m] / 256 (the k = 1 lanes give zero)
        const float swk = swl[swr + k] * (1.0f / 256.0f);
        const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : swk, lh ? 0.0f : sa[k], zf, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            y[e] = __builtin_fmaf((float)acc[e], S[e], y[e]);
    };

    // ---- INT4 tiles: up to SLOTS pairs in flight; the loop is unrolled (the
    // token scales of tile k sit in registers sa[k], the weight scales in LDS)
#pragma unroll
    for (int j = 0; j < MAXT / 2; ++j) {
        if (j < np) {
            compiler_fence();
            wait_pairs(min(np - 1 - j, SLOTS - 1));           // later pairs may stay in flight
            compiler_fence();
            const unsigned char *sl = wl + (j % SLOTS) * WSLOT;
            tile(sl, 0, 2 * j);
            if (2 * j + 1 < nt)
                tile(sl, 1, 2 * j + 1);
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));       // this slot's reads are back
            compiler_fence();
            if (j + SLOTS < np)
                issue(j + SLOTS);
        }
    }

    // ---- INT8 tail: wave w < T8 takes tail tile w (folded once) ----------------------
    if (tail_wave) {
        const uint4 tx0 = *reinterpret_cast<const uint4 *>(tail + mrow * kTileBytes + 16 * lh);
        const uint4 tx1 = *reinterpret_cast<const uint4 *>(tail + mrow * kTileBytes + 32 + 16 * lh);
        v16i acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[0]), as_v4i(tx0), zi, 0, 0, 0);
        acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(tw[1]), as_v4i(tx1), acc8, 0, 0, 0);
        const v16f S = __builtin_amdgcn_mfma_f32_32x32x2f32(lh ? 0.0f : a.sw8[nrow], lh ? 0.0f : t8s[mrow], zf,
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

}  // namespace decode_fused_impl

using namespace decode_fused_impl;

bool decode_fused_fits(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    if (K > 32768)
        return false;                                         // the exact sum of squares stays below 2^95
    const int32_t K_n = K - n_out;
    if (M < 1 || M > MAXM || group != 128 || K_n < 128 || K_n % 128 != 0 || n_out < 0 || n_out > MAXOUT)
        return false;
    const int T4 = K_n / 128;
    if ((T4 + WAVES - 1) / WAVES > MAXT)
        return false;
    // DMA offsets are 32-bit: every packed weight row must start below 4 GiB
    return (int64_t)N * T4 * kTileBytes < (int64_t(1) << 32);
}

hipError_t launch_decode_fused(const DecodeFusedArgs &a, hipStream_t stream) {
    if (a.gamma)
        hipLaunchKernelGGL(decode_fused_kernel<true>, dim3((a.N + BN - 1) / BN), dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_fused_kernel<false>, dim3((a.N + BN - 1) / BN), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
