// FP6 GEMM for group scales of 128 channels (the 128 x 128 kernel).
#include <algorithm>

#include "w4a4.h"
#include "gemm_fp6_common.h"
#include "gemm_fp6_internal.h"

namespace w4a4 {
namespace gemm_fp6_impl {

// ---------------------------------------------------------------------------
// Group scales of 128 channels: one scale per (row, group) on both operands,
// y = sum over groups g of (sa[m, g] sw[n, g]) * acc_g[m, n] (Atom summary
// page, Summary paragraph 2 and Key points item 5). A group is two FP6 k-steps.
// * The fold y += acc_g * (sa sw) costs the VALU one FMA per output element
//   and group, as much time as the group's FP6 MFMAs: the two have to run
//   side by side. 128 x 128 output tile per workgroup, four waves of 64 x 64
//   (2 x 2 blocks), and two workgroups per CU (under 80 KB of LDS each), so
//   each SIMD holds one wave of each: the two workgroups pass their barriers
//   independently, and one's fold or fragment reads overlap the other's
//   MFMAs. Per wave the group sums (64) and y (64) both in VGPRs, so the fold
//   reads the sums directly.
// * Per group: the eight fragment reads of both k-steps, then for each pair of
//   blocks the scale products of the previous group (one
//   v_mfma_f32_32x32x1_2b_f32: exact fp32 outer products of row and column
//   scales, in the accumulator layout), the fold of that group's sums, and
//   this group's two k-steps into the same registers (C = 0 on the first).
// * Ring of three stages of one group each (both k-steps of A and B), two
//   groups ahead; the group scales of four groups at a time in a double
//   buffer beside it, requested with the first group of their block; the
//   previous group's scales are kept in registers for its fold.
// * The INT8 tail and the epilogue as in the 256 x 256 kernel:
//   Y = fp16(y + acc8 * (sa8 sw8)).
constexpr int kGThreads = 256;
constexpr int GBM = 128, GBN = 128, GWT = 64, GF = 2;
constexpr int GSTAGES = 3;
constexpr int G_A = 0;                              // A: k-step s, block i at s * 4 BLK + i BLK
constexpr int G_B = 2 * (GBM / 32) * BLK;           // B: k-step s, block i at G_B + s * 4 BLK + i BLK
constexpr int GSTAGE = G_B + 2 * (GBN / 32) * BLK;  // 24576 bytes
constexpr int G_DA = 2 * (GBM / 32) * BLK / 16 / kGThreads;  // 3 DMA units of A per group per lane
constexpr int G_DB = 2 * (GBN / 32) * BLK / 16 / kGThreads;  // 3 of B
constexpr int G_D = G_DA + G_DB;                    // 6 per lane (+ 4 scale units every G_SB groups)
constexpr int G_TAIL_TILE = (GBM + GBN) * kTileBytes;   // 16 KB
// Group scales go in blocks of G_SB groups: rows [128][G_SB], then columns
// [128][G_SB], two blocks (double buffer) after the ring. After the loop the
// first block holds the tail scales sa8[128], sw8[128] of the tile.
constexpr int G_SB = 4;
constexpr int G_SBUF = G_SB * (GBM + GBN) * 4;      // 4 KB
constexpr int G_SCB = GSTAGES * GSTAGE;
constexpr int G_SCALES8 = G_SCB;
constexpr int G_LDS_BYTES = G_SCB + 2 * G_SBUF;     // 80 KB: two workgroups per CU
constexpr int G_YP = 2 * GBN + 16;                  // bytes per row of the staged fp16 tile
static_assert(GBM * G_YP <= G_SCB, "the staged tile fits the ring");
static_assert(G_DA == 3 && G_DB == 3 && GBM + GBN == kGThreads, "whole DMA rounds");
static_assert(2 * G_LDS_BYTES <= 160 * 1024, "two workgroups per CU");
static_assert(MAX_TAIL_TILES * G_TAIL_TILE <= G_SCB, "the tail fits the ring");

// FP6 MFMA (operands FP6 E2M3 holding q / 8, block scale 2^3 on each):
// acc += w^T x, and acc = w^T x. Written as instructions so that every
// register stays an architectural VGPR (the fold reads the sums with no AGPR
// copies); block (fm, fn) takes the weight fragment as the first operand, so
// lane (li, lh) holds token row li and the columns 8 (r / 4) + 4 lh + r % 4.
__device__ __forceinline__ void mma(v16f &acc, const v6i &w, const v6i &x) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:2 blgp:2"
                 : "+v"(acc)
                 : "v"(w), "v"(x), "v"(130));
}
__device__ __forceinline__ void mma0(v16f &acc, const v6i &w, const v6i &x) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0] cbsz:2 blgp:2"
                 : "=&v"(acc)
                 : "v"(w), "v"(x), "v"(130));
}

__device__ __forceinline__ float y_value_g(float yh, int acc8, float s8) {
#pragma clang fp contract(off)
    float y = __builtin_fmaf((float)acc8, s8, yh);
    asm volatile("" : "+v"(y));
    return y;
}

template <bool EXPORT>
__global__ __launch_bounds__(kGThreads) void gemm_fp6_group_kernel(Fp6GemmArgs a) {
    __shared__ __align__(16) unsigned char lds[G_LDS_BYTES];
    const float *sS8 = reinterpret_cast<const float *>(lds + G_SCALES8);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;          // 2 x 2 waves of 64 x 64
    const int li = lane & 31, lh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    const int tiles_m = (a.M + GBM - 1) / GBM, tiles_n = (a.N + GBN - 1) / GBN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    const int row0 = tm * GBM, col0 = tn * GBN;

    const int RBA = (a.M + 31) / 32, RBB = (a.N + 31) / 32;
    const int T = (int)(a.pitch4 / 32);            // head K-tiles of 64 channels
    const int G = T / 2;                           // groups of 128 channels
    const int T8 = (int)(a.pitch8 / kTileBytes);

    // DMA sources. A and B alike: unit q = j * 256 + tid (768 per group),
    // k-step q / 384, block (q % 384) / 96, 16-byte unit q % 96. Scales: a
    // block of G_SB groups with the first group of the block, unit u =
    // i * 256 + tid of each table being row (or column) u / G_SB, group
    // u % G_SB: a wave's 64 units are the G_SB consecutive floats of 16 rows
    // (16 cache lines, where one scale per row per group would touch 64).
    uint32_t oa[G_DA], ob[G_DB];
#pragma unroll
    for (int j = 0; j < G_DA; ++j) {
        const int q = j * kGThreads + tid, s = q / 384, i = (q % 384) / 96, u = q % 96;
        oa[j] = ((uint32_t)min(row0 / 32 + i, RBA - 1) * (uint32_t)T + (uint32_t)s) * (uint32_t)BLK + 16 * u;
        ob[j] = ((uint32_t)min(col0 / 32 + i, RBB - 1) * (uint32_t)T + (uint32_t)s) * (uint32_t)BLK + 16 * u;
    }
    const bool low = wave_u < 2;                   // uniform per wave
    const int64_t srow = min(row0 + (tid & (GBM - 1)), a.M - 1), scol = min(col0 + (tid & (GBN - 1)), a.N - 1);
    // ring group gg (past the last: a reload of the last into a stage nothing reads)
    auto issue = [&](int gg) {
        const int g = min(gg, G - 1);
        const uint32_t st = lds_addr(lds) + (gg % GSTAGES) * GSTAGE;
        const uint8_t *A = a.a_u6 + (int64_t)(2 * g) * BLK, *B = a.w_u6 + (int64_t)(2 * g) * BLK;
#pragma unroll
        for (int j = 0; j < G_DA; ++j)
            dma16(A, oa[j], st + G_A + j * 4096 + wave_u * 1024);
#pragma unroll
        for (int j = 0; j < G_DB; ++j)
            dma16(B, ob[j], st + G_B + j * 4096 + wave_u * 1024);
        if (gg % G_SB == 0) {                       // uniform: the scale block of groups gg ..
            const uint32_t sb = lds_addr(lds) + G_SCB + ((gg / G_SB) & 1) * G_SBUF;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int u = i * kGThreads + tid, r = u / G_SB, gk = min(gg + u % G_SB, G - 1);
                dma4(a.sa4 + (int64_t)min(row0 + r, a.M - 1) * G + gk, sb + i * 1024 + wave_u * 256);
                dma4(a.sw4 + (int64_t)min(col0 + r, a.N - 1) * G + gk, sb + GBM * G_SB * 4 + i * 1024 + wave_u * 256);
            }
        }
    };

    float y[GF][GF][16];
#pragma unroll
    for (int fm = 0; fm < GF; ++fm)
#pragma unroll
        for (int fn = 0; fn < GF; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                y[fm][fn][r] = 0.0f;
    v16f acc[GF][GF];

    // fragment reads: lane (li, lh) reads chunk lh of row li of a block
    const uint32_t llo = 512 * lh + 16 * li, lhi = 1024 + 256 * lh + 8 * li;
    uint32_t ha[2][GF], hb[2][GF];                // 8-byte reads on bases of their own (not merged)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < GF; ++i) {
            ha[s][i] = G_A + (s * 4 + wm * 2 + i) * BLK + lhi;
            hb[s][i] = G_B + (s * 4 + wn * 2 + i) * BLK + lhi;
            asm("" : "+v"(ha[s][i]));
            asm("" : "+v"(hb[s][i]));
        }

    // y += acc * S for one block; S = the half of a scale product that
    // belongs to it. Export (test path): the group's exact integer sums.
    auto fold = [&](int fm, int fn, const v32f &S, int half, int g) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            y[fm][fn][r] = __builtin_fmaf(acc[fm][fn][r], S[16 * half + r], y[fm][fn][r]);
        if constexpr (EXPORT) {
            const int m = row0 + wm * GWT + fm * 32 + li;
            if (m < a.M) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = col0 + wn * GWT + fn * 32 + lh * 4 + (r / 4) * 8 + (r % 4);
                    if (n < a.N)
                        a.acc4_out[((int64_t)g * a.M + m) * a.N + n] = (int32_t)acc[fm][fn][r];
                }
            }
        }
    };

#pragma unroll
    for (int p = 0; p < 2; ++p)
        issue(p);
    // scales of the previous group: row scale of block fm = lh, column scales
    // of blocks fn = lh and 1 - lh (row / column li)
    float prs = 0.0f, pca = 0.0f, pcb = 0.0f;
    for (int g = 0; g < G; ++g) {
        compiler_fence();
        // group g has landed (g + 1, and the scale block that comes with it, may not)
        if ((g + 1) % G_SB == 0)
            __builtin_amdgcn_s_waitcnt(vmcnt_only(G_D + 4));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_only(G_D));
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        // every wave is done with group g - 1's stage: group g + 2 goes there.
        // The sums of g - 1 (written by MFMAs the compiler does not see as
        // such) get their wait states before the folds read them.
        issue(g + 2);
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        const uint32_t st = (uint32_t)((g % GSTAGES) * GSTAGE);
        v6i fa[2][GF], fb[2][GF];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < GF; ++i) {
                fa[s][i] = load_operand(lds + st + G_A + (s * 4 + wm * 2 + i) * BLK + llo, lds + st + ha[s][i]);
                fb[s][i] = load_operand(lds + st + G_B + (s * 4 + wn * 2 + i) * BLK + llo, lds + st + hb[s][i]);
            }
        const float *sc = reinterpret_cast<const float *>(lds + G_SCB + ((g / G_SB) & 1) * G_SBUF) + g % G_SB;
        const float crs = sc[(wm * GWT + lh * 32 + li) * G_SB];
        const float cca = sc[(GBM + wn * GWT + lh * 32 + li) * G_SB];
        const float ccb = sc[(GBM + wn * GWT + (1 - lh) * 32 + li) * G_SB];
        // pair c: blocks (0, c) in the first half of S, (1, c) in the second;
        // the two MFMAs of each k-step share the weight fragment, so fewer
        // operand bits change between consecutive MFMAs
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (g > 0) {
                const v32f z = {};
                const v32f S = __builtin_amdgcn_mfma_f32_32x32x1f32((c ^ lh) ? pcb : pca, prs, z, 0, 0, 0);
                fold(0, c, S, 0, g - 1);
                fold(1, c, S, 1, g - 1);
            }
            mma0(acc[0][c], fb[0][c], fa[0][0]);
            mma0(acc[1][c], fb[0][c], fa[0][1]);
            mma(acc[0][c], fb[1][c], fa[1][0]);
            mma(acc[1][c], fb[1][c], fa[1][1]);
        }
        prs = crs, pca = cca, pcb = ccb;
    }
    // the last group's fold
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const v32f z = {};
        const v32f S = __builtin_amdgcn_mfma_f32_32x32x1f32((c ^ lh) ? pcb : pca, prs, z, 0, 0, 0);
        fold(0, c, S, 0, G - 1);
        fold(1, c, S, 1, G - 1);
    }

    // ---- the INT8 tail, staged into the ring once every wave is done with it -----------
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (T8 > 0) {
        {                                                          // tail scales into the first scale block
            const uint32_t ss = lds_addr(lds) + G_SCALES8;
            if (low)
                dma4(a.sa8 + srow, ss + wave_u * 256);
            else
                dma4(a.sw8 + scol, ss + wave_u * 256);
        }
#pragma unroll
        for (int j = 0; j < MAX_TAIL_TILES; ++j) {
            if (j >= T8)
                break;                                             // uniform
            const uint32_t st = lds_addr(lds) + j * G_TAIL_TILE + wave_u * 1024;
            const uint8_t *A8 = reinterpret_cast<const uint8_t *>(a.a8) + j * kTileBytes;
            const uint8_t *B8 = reinterpret_cast<const uint8_t *>(a.w8) + j * kTileBytes;
            // 128 rows of 64 bytes per operand: two units of 16 bytes per lane each
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int q = k * kGThreads + tid, r = q >> 2;
                dma16(A8, (uint32_t)min(row0 + r, a.M - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q), st + k * 4096);
                dma16(B8, (uint32_t)min(col0 + r, a.N - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q),
                      st + GBM * kTileBytes + k * 4096);
            }
        }
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    }

    // ---- epilogue: tail sums and final values (packed fp16), then Y through LDS ---------
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t yp[GF][GF][8];
#pragma unroll
    for (int fn = 0; fn < GF; ++fn) {
        const int nl = wn * GWT + fn * 32 + lh * 4;       // tile-local first column of the lane
#pragma unroll
        for (int fm = 0; fm < GF; ++fm) {
            const int ml = wm * GWT + fm * 32 + li;
            const int m = row0 + ml;
            v16i acc8 = zi;
#pragma unroll
            for (int j = 0; j < MAX_TAIL_TILES; ++j) {
                if (j >= T8)
                    break;                                 // uniform
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint4 pb = *reinterpret_cast<const uint4 *>(lds + j * G_TAIL_TILE + GBM * kTileBytes +
                                                                     swz(wn * GWT + fn * 32 + li, 2 * s + lh));
                    const uint4 p = *reinterpret_cast<const uint4 *>(lds + j * G_TAIL_TILE + swz(ml, 2 * s + lh));
                    acc8 = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{(int)pb.x, (int)pb.y, (int)pb.z, (int)pb.w},
                                                                 v4i{(int)p.x, (int)p.y, (int)p.z, (int)p.w},
                                                                 acc8, 0, 0, 0);
                }
            }
            if constexpr (EXPORT) {
                if (m < a.M && a.acc8_out) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int n = col0 + nl + (r / 4) * 8 + (r % 4);
                        if (n < a.N)
                            a.acc8_out[(int64_t)m * a.N + n] = acc8[r];
                    }
                }
            }
            const float rs8 = T8 > 0 ? sS8[ml] : 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 c8v = *reinterpret_cast<const float4 *>(sS8 + GBM + nl + q * 8);
                const float4 c8 = T8 > 0 ? c8v : float4{0.0f, 0.0f, 0.0f, 0.0f};
                const float cs8[4] = {c8.x, c8.y, c8.z, c8.w};
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = y_value_g(y[fm][fn][q * 4 + e], acc8[q * 4 + e], rs8 * cs8[e]);
                yp[fm][fn][2 * q] = pack_half2(v[0], v[1]);
                yp[fm][fn][2 * q + 1] = pack_half2(v[2], v[3]);
            }
        }
    }

    // Every wave is done with the tail tiles: the tile's fp16 values go to
    // rows of G_YP bytes at the start of the ring, and from there to Y as
    // 16-byte pieces of whole rows (a store instruction writes four rows of
    // 256 bytes instead of 32 pieces of 16 bytes).
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
#pragma unroll
    for (int fn = 0; fn < GF; ++fn)
#pragma unroll
        for (int fm = 0; fm < GF; ++fm) {
            unsigned char *yrow = lds + (wm * GWT + fm * 32 + li) * G_YP + 2 * (wn * GWT + fn * 32 + lh * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2 *>(yrow + 16 * q) = uint2{yp[fm][fn][2 * q], yp[fm][fn][2 * q + 1]};
        }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    const uintptr_t ya = reinterpret_cast<uintptr_t>(a.y) | (uintptr_t)(a.ldy * 2);
    constexpr int RPP = kGThreads / 16;                  // 16 lanes per row: rows per pass
    const int rr = tid >> 4, ch = tid & 15;
    if (row0 + GBM <= a.M && col0 + GBN <= a.N && (ya & 15) == 0) {      // uniform: no checks
        uint4 v[GBM / RPP];
#pragma unroll
        for (int p = 0; p < GBM / RPP; ++p)
            v[p] = *reinterpret_cast<const uint4 *>(lds + (p * RPP + rr) * G_YP + 16 * ch);
        _Float16 *dst = a.y + (int64_t)(row0 + rr) * a.ldy + col0 + ch * 8;
#pragma unroll
        for (int p = 0; p < GBM / RPP; ++p)
            *reinterpret_cast<uint4 *>(dst + (int64_t)(p * RPP) * a.ldy) = v[p];
        return;
    }
#pragma unroll
    for (int p = 0; p < GBM / RPP; ++p) {
        const int ml = p * RPP + rr, m = row0 + ml, n = col0 + ch * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(lds + ml * G_YP + 16 * ch);
        if (m >= a.M)
            continue;
        _Float16 *dst = a.y + (int64_t)m * a.ldy + n;
        if (n + 7 < a.N && (ya & 15) == 0) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else if (n + 7 < a.N && (ya & 7) == 0) {
            reinterpret_cast<uint2 *>(dst)[0] = uint2{v.x, v.y};
            reinterpret_cast<uint2 *>(dst)[1] = uint2{v.z, v.w};
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < a.N)
                    reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
        }
    }
}

}  // namespace gemm_fp6_impl

hipError_t launch_gemm_fp6_group(const Fp6GemmArgs &a, bool export_acc, hipStream_t stream) {
    using namespace gemm_fp6_impl;
    const int tiles = ((a.M + GBM - 1) / GBM) * ((a.N + GBN - 1) / GBN);
    if (export_acc)
        hipLaunchKernelGGL(gemm_fp6_group_kernel<true>, dim3(tiles), dim3(kGThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_fp6_group_kernel<false>, dim3(tiles), dim3(kGThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
