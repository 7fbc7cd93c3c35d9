// Prefill GEMM on the FP6 matrix cores: INT4 x INT4 head with each INT4 code
// q held as the FP6 E2M3 value q / 8, exact fp32 accumulation; INT8 x INT8 outlier tail
// on the i8 matrix cores; fp32 scale epilogue to fp16.
//
// Method: Atom summary page (Summary paragraph 2: INT4 main part plus an
// 8-bit outlier part over reordered channels; Key points item 5: symmetric
// scales factor out of the integer sums) and the QUIK abstract (hybrid 4-bit
// layer with higher-precision outliers). The integer sums are those of the
// i8 kernels; only the matrix instruction that forms them differs.
//
// CDNA4 design
// * CDNA4 has no INT4 matrix instruction, but its FP6 one
//   (v_mfma_scale_f32_32x32x64_f8f6f4) runs at twice the i8 rate. E2M3 holds
//   q / 8 exactly for every INT4 code (the multiples of 1/8 up to 1 in
//   magnitude: subnormals below 1, so the code is |q| with a sign bit), and
//   the instruction's block scale 2^3 on each operand gives back q: every product is the integer qa qw (below 2^7) and every partial
//   sum an integer below 2^24 in magnitude (|sum| <= 64 K_n), so the fp32
//   accumulator holds the exact integer sum whatever order the matrix core
//   adds in; the accumulator export converts it to int32 unchanged. (E3M2,
//   which holds q itself, and E2M3 of q / 2 are exact too. The matrix core's
//   power, and with it the clock, depends on the operand bits: E2M3 of q / 2
//   ran about 5% faster than E3M2 of q, and E2M3 of q / 8, whose codes are
//   the small integers |q|, about 1.5% faster again.)
// * The FP6 operand of a lane is a 192-bit image of 32 codes (code i at bits
//   6i). Unpacking nibbles into it costs more VALU per MFMA than the FP6
//   rate leaves, so the operands arrive already in that form, in a "u6"
//   layout built for this kernel: 32-row x 64-channel blocks of 1536
//   contiguous bytes, each laid out as LDS wants it (row r's chunk h: image
//   bytes 0..15 at 512 h + 16 r, bytes 16..23 at 1024 + 256 h + 8 r). A DMA
//   instruction then moves whole cache lines, and the b128 / b64 fragment
//   reads of 16 lanes cover 128 contiguous bytes (no bank conflicts).
//   repack_u6_kernel converts packed nibbles to it (once for weights; per
//   call for activations).
// * 256 x 256 output tile per workgroup, four waves of 128 x 128 (4 x 4
//   blocks of 32 x 32), fp32 accumulators in AGPRs, one wave per SIMD. A
//   K-tile is 64 channels (one FP6 k-step): eight u6 blocks of each operand,
//   24 KB per stage; a 6-stage ring, DMA five tiles ahead, one barrier per
//   tile. The fragments of tile t + 1 are read from LDS into a second
//   register set while the sixteen MFMAs of tile t run.
// * The INT8 tail (at most 256 channels) is staged into the ring once the
//   head is done and multiplied block by block on the i8 matrix cores into a
//   16-register int32 accumulator; y = fp16(acc4 * (sa4 sw4) + acc8 * (sa8
//   sw8)).
#include <algorithm>
#include <type_traits>

#include "w4a4.h"
#include "gemm_fp6_common.h"
#include "gemm_fp6_internal.h"

namespace w4a4 {
namespace gemm_fp6_impl {

// ---------------------------------------------------------------------------
// repack: packed two's complement nibbles -> u6 planes
// ---------------------------------------------------------------------------

// E2M3 code of q / 8 for a two's complement nibble q (code = s << 5 | e << 3
// | m, value 2^(e-1) (1 + m/8), subnormal m/8): |q| / 8 for |q| = 1..7 is the
// subnormal m = |q|, and 8 / 8 = 2^0 is e = 1, m = 0, so the code is |q| with
// the sign in bit 5.
__device__ __forceinline__ uint32_t e2m3_of_nibble(uint32_t n) {
    const uint32_t neg = (n >> 3) & 1;
    const uint32_t mag = neg ? 16u - n : n;                  // |q| of the two's complement nibble
    return (neg << 5) | mag;
}

// One lane per (row, 64-channel tile): 32 nibble bytes in, the two chunk
// images out. Lanes are ordered row-fastest inside a 32-row block, so the
// image stores of consecutive lanes are consecutive; rows past the last one
// of the operand are written as code 0.
__global__ __launch_bounds__(256) void repack_u6_kernel(const uint8_t *q4, int64_t rows, int64_t pitch4,
                                                         uint8_t *u6) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t T = pitch4 / 32, RB = (rows + 31) / 32;
    const int64_t total = RB * T * 32;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t rr = i & 31, bt = i >> 5;            // row inside the block, block index
        const int64_t b = bt / T, t = bt % T;
        const int64_t r = b * 32 + rr;
        unsigned char *blk = u6 + bt * kU6Block;           // block (b, t) is block b * T + t
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t w[6] = {0, 0, 0, 0, 0, 0};
            if (r < rows) {
                const u32x4 p = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(q4 + r * pitch4 + t * 32 + h * 16));
                const uint32_t pw[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const uint32_t code = e2m3_of_nibble((pw[j >> 3] >> (4 * (j & 7))) & 15);
                    const int bit = 6 * j, d = bit >> 5, off = bit & 31;
                    w[d] |= code << off;
                    if (off > 26)
                        w[d + 1] |= code >> (32 - off);
                }
            }
            *reinterpret_cast<uint4 *>(blk + 512 * h + 16 * rr) = uint4{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<uint2 *>(blk + 1024 + 256 * h + 8 * rr) = uint2{w[4], w[5]};
        }
    }
}

// ---------------------------------------------------------------------------
// 256 x 256 FP6 GEMM for one scale per row (group 0)
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128, FM = 4, FN = 4;
constexpr int STAGES = 6;                          // ring depth
constexpr int A_OFF = 0, B_OFF = (BM / 32) * BLK;  // eight blocks of each operand per stage
constexpr int STAGE = B_OFF + (BN / 32) * BLK;     // 24 KB
constexpr int DPO = (BM / 32) * BLK / 16 / kThreads;   // DMA instructions per operand per K-tile
constexpr int D = 2 * DPO;                         // DMA instructions per K-tile per lane
constexpr int TAIL_TILE = (BM + BN) * kTileBytes;  // 32 KB: A rows, then B rows (swizzled 64-byte rows)
constexpr int SCALES = STAGES * STAGE;             // sa4, sa8, sw4, sw8 of the tile
constexpr int LDS_BYTES = SCALES + 4 * BM * 4;
static_assert(MAX_TAIL_TILES * TAIL_TILE <= STAGES * STAGE, "the tail fits in the ring");
constexpr int Y_ROW = 80;                          // bytes per staged row of a 32 x 32 fp16 block
constexpr int Y_SLOTS = STAGES * STAGE - (kThreads / 64) * 32 * Y_ROW;   // one slot per wave
static_assert(MAX_TAIL_TILES * TAIL_TILE <= Y_SLOTS, "the slots stay clear of the tail");
static_assert(STAGE == 24576 && DPO == 3, "stage layout");
static_assert((STAGES - 1) * D <= 63, "vmcnt range");

// acc += w^T x for one 32 x 32 block (both operands FP6 E2M3 holding q / 8,
// block scale exponent 130 = 2^3 on each).
// Block (fm, fn) takes the weight fragment as the first operand, so lane
// (li, lh) holds token row li and the columns 8 (r / 4) + 4 lh + r % 4.
// Written as an instruction so that the accumulators stay in AGPRs and the
// fragments in VGPRs with no copies; the compiler places the waits for the
// fragments' LDS reads in front of it, but not the two wait states an MFMA
// needs after a VALU write of its operands. Here the operands come straight
// from LDS reads (no moves in the main loop, whose first MFMA follows the
// barrier and the DMA issue); the MFMAs elsewhere in these kernels, whose
// operands the compiler may form with moves, carry an s_nop 1 of their own.
__device__ __forceinline__ void mma(v16f &acc, const v6i &w, const v6i &x) {
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:2 blgp:2"
                 : "+a"(acc)
                 : "v"(w), "v"(x), "v"(130));
}

// acc8 += w^T x and acc8 = w^T x on the i8 matrix core (the INT8 tail),
// written as instructions so that the sums stay in VGPRs: the AGPRs hold the
// head's sums.
__device__ __forceinline__ void mma_i8(v16i &acc, const v4i &w, const v4i &x) {
    asm volatile("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(acc) : "v"(w), "v"(x));
}
__device__ __forceinline__ void mma_i8_0(v16i &acc, const v4i &w, const v4i &x) {
    asm volatile("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, 0" : "=&v"(acc) : "v"(w), "v"(x));
}

// y = acc4 * s4 + acc8 * s8: one product, one fused multiply-add, rounded to
// fp32 before the fp16 conversion (the same bits in every launch).
__device__ __forceinline__ float y_value(float acc4, int acc8, float s4, float s8) {
#pragma clang fp contract(off)
    const float p4 = acc4 * s4;
    float y = __builtin_fmaf((float)acc8, s8, p4);
    asm volatile("" : "+v"(y));
    return y;
}

template <bool EXPORT>
__global__ __launch_bounds__(kThreads) void gemm_fp6_big_kernel(Fp6GemmArgs a) {
    __shared__ __align__(16) unsigned char lds[LDS_BYTES];
    float *sS = reinterpret_cast<float *>(lds + SCALES);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, true, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    // ---- DMA sources of this lane (fixed for the K loop) -------------------------
    // A stage holds the eight 32-row blocks of each operand for one K-tile,
    // copied whole: unit q = j * 256 + tid of an operand is bytes 16 (q % 96)
    // of block q / 96 (clamped to the last block of the operand).
    const int RBA = (a.M + 31) / 32, RBB = (a.N + 31) / 32;
    const int T = (int)(a.pitch4 / 32);            // head K-tiles of 64 channels
    const int T8 = (int)(a.pitch8 / kTileBytes);   // tail K-tiles of 64 INT8 channels
    uint32_t oa[DPO], ob[DPO];
#pragma unroll
    for (int j = 0; j < DPO; ++j) {
        const int q = j * kThreads + tid, i = q / 96, u = q % 96;
        oa[j] = (uint32_t)min(row0 / 32 + i, RBA - 1) * (uint32_t)(T * BLK) + 16 * u;
        ob[j] = (uint32_t)min(col0 / 32 + i, RBB - 1) * (uint32_t)(T * BLK) + 16 * u;
    }

    // ring tile tt (past the last head tile: a reload of the last one into a
    // stage nothing reads again, so every iteration issues the same DMA);
    // part j < DPO is unit j of A, part DPO + j unit j of B
    auto issue_part = [&](int tt, int j) {
        const int t = min(tt, T - 1);
        const uint32_t st = lds_addr(lds) + (tt % STAGES) * STAGE + wave_u * 1024;
        if (j < DPO)
            dma16(a.a_u6 + (int64_t)t * BLK, oa[j], st + A_OFF + j * 4096);
        else
            dma16(a.w_u6 + (int64_t)t * BLK, ob[j - DPO], st + B_OFF + (j - DPO) * 4096);
    };
    auto issue = [&](int tt) {
#pragma unroll
        for (int j = 0; j < D; ++j)
            issue_part(tt, j);
    };

    // ---- scales of the tile, ahead of every K-tile (the first wait covers them)
    {
        const uint32_t ss = lds_addr(sS) + wave_u * 256;
        const int64_t mr = min(row0 + tid, a.M - 1), nc = min(col0 + tid, a.N - 1);
        dma4(a.sa4 + mr, ss);
        dma4(a.sw4 + nc, ss + 2 * BM * 4);
        if (T8 > 0) {
            dma4(a.sa8 + mr, ss + BM * 4);
            dma4(a.sw8 + nc, ss + 3 * BM * 4);
        }
    }

    v16f acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[fm][fn][r] = 0.0f;

    // Per-lane LDS offsets of this wave's fragments inside a stage: lane
    // (li, lh) of row block i reads chunk lh of row li of block 4 wm + i (A)
    // or 4 wn + i (B); a row block adds BLK bytes (an immediate offset).
    const uint32_t la = A_OFF + (wm * 4) * BLK, lb = B_OFF + (wn * 4) * BLK;
    const uint32_t llo = 512 * lh + 16 * li, lhi = 1024 + 256 * lh + 8 * li;
    // The 8-byte reads each get a base register of their own: two of them a
    // block apart on one base would be merged into a single four-register
    // read, which cannot land inside two operand tuples.
    uint32_t ha[FM], hb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        ha[i] = la + lhi + i * BLK;
        asm("" : "+v"(ha[i]));
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        hb[i] = lb + lhi + i * BLK;
        asm("" : "+v"(hb[i]));
    }
    auto a_frag = [&](uint32_t st, int i) {
        return load_operand(lds + st + la + llo + i * BLK, lds + st + ha[i]);
    };
    auto b_frag = [&](uint32_t st, int i) {
        return load_operand(lds + st + lb + llo + i * BLK, lds + st + hb[i]);
    };

    // ---- head -------------------------------------------------------------------------
    // Register double buffer: at the top of tile t the registers hold all
    // eight fragments of tile t. After the barrier that has every wave holding
    // tile t (so its stage is free) and tile t + 1 landed, tile t + 6 goes into
    // tile t's stage, the sixteen reads of tile t + 1 are issued, and the
    // sixteen MFMAs of tile t run while they are in flight.
#pragma unroll
    for (int p = 0; p < STAGES; ++p)
        issue(p);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only((STAGES - 1) * D));     // tile 0 (and the scales)
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    v6i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
        fa0[i] = a_frag(0, i);
#pragma unroll
    for (int i = 0; i < FN; ++i)
        fb0[i] = b_frag(0, i);

    auto tile = [&](int t, const v6i (&xa)[FM], const v6i (&xb)[FN], v6i (&na)[FM], v6i (&nb)[FN]) {
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(vmcnt_only((STAGES - 2) * D));   // tile t + 1 has landed
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));               // tile t is in registers
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        // The sixteen MFMAs of tile t, each followed by one fragment read of
        // tile t + 1 (the first eight) or one DMA unit of tile t + 6 into tile
        // t's stage (the next six), so that every other instruction issues
        // while an MFMA executes. The blocks go in serpentine order (fn
        // forward for even fm, backward for odd), so that consecutive MFMAs
        // share one operand: fewer operand bits change from one MFMA to the
        // next, the matrix core draws less power, and at the clock that power
        // allows the kernel ran about 2% faster than in row order.
        const uint32_t sn = (uint32_t)(((t + 1) % STAGES) * STAGE);
#pragma unroll
        for (int k = 0; k < FM * FN; ++k) {
            const int fm = k / FN, fn = fm % 2 == 0 ? k % FN : FN - 1 - k % FN;
            mma(acc[fm][fn], xb[fn], xa[fm]);
            if (k < FM)
                na[k] = a_frag(sn, k);
            else if (k < FM + FN)
                nb[k - FM] = b_frag(sn, k - FM);
            else if (k < FM + FN + D)
                issue_part(t + STAGES, k - FM - FN);
        }
    };
    for (int t = 0; t < T; t += 2) {
        tile(t, fa0, fb0, fa1, fb1);
        if (t + 1 < T)
            tile(t + 1, fa1, fb1, fa0, fb0);
    }

    // The MFMAs above are instructions the compiler does not see as such: give
    // the last ones the wait states their AGPR results need before the VALU
    // reads them.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // ---- the INT8 tail: staged into the ring once every wave is done with it ----------
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (T8 > 0) {
        // tail tile j: A rows at j * TAIL_TILE, B rows after them; 16-byte
        // chunk c of row r at swz(r, c), lane q of a DMA instruction row q / 4
#pragma unroll
        for (int j = 0; j < MAX_TAIL_TILES; ++j) {
            if (j >= T8)
                break;                                             // uniform
            const uint32_t st = lds_addr(lds) + j * TAIL_TILE + wave_u * 1024;
            const uint8_t *A8 = reinterpret_cast<const uint8_t *>(a.a8) + j * kTileBytes;
            const uint8_t *B8 = reinterpret_cast<const uint8_t *>(a.w8) + j * kTileBytes;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int q = k * kThreads + tid, r = q >> 2;
                dma16(A8, (uint32_t)min(row0 + r, a.M - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q), st + k * 4096);
                dma16(B8, (uint32_t)min(col0 + r, a.N - 1) * (uint32_t)a.pitch8 + dma_chunk_offset(q),
                      st + BM * kTileBytes + k * 4096);
            }
        }
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    }

    // ---- epilogue, a column of four blocks at a time ---------------------------------
    // The four tail sums of a column are independent MFMA chains, issued side
    // by side. Lane coordinates are taken afresh here so that nothing derived
    // from them has to stay live (or spill) across the main loop.
    uint32_t tid_e = threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int lane_e = (int)(tid_e & 63), wave_e = (int)(tid_e >> 6);
    const int wm_e = wave_e >> 1, wn_e = wave_e & 1, li_e = lane_e & 31, lh_e = lane_e >> 5;
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const bool vec_store = ((reinterpret_cast<uintptr_t>(a.y) | (uintptr_t)(a.ldy * 2)) & 7) == 0;
    const bool interior = ((reinterpret_cast<uintptr_t>(a.y) | (uintptr_t)(a.ldy * 2)) & 15) == 0 &&
                          row0 + BM <= a.M && col0 + BN <= a.N;
    // Two copies of the epilogue: one for tiles wholly inside Y (no checks),
    // one for the edge tiles, each contiguous, so that a tile fetches only the
    // instructions it runs (the unrolled epilogue is most of the kernel's code).
    auto epilogue = [&](auto interior_tag) {
    constexpr bool INTERIOR = decltype(interior_tag)::value;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int nl = wn_e * WTN + fn * 32 + lh_e * 4;   // tile-local first column of the lane
        v16i acc8[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            acc8[fm] = zi;                                 // (kept when there is no tail)
        // all ten fragment reads of a tail tile are issued before its eight
        // MFMAs (one LDS round trip per tile, not one per MFMA)
#pragma unroll
        for (int j = 0; j < MAX_TAIL_TILES; ++j) {
            if (j >= T8)
                break;                                     // uniform
            v4i b8[2], a8[2][FM];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                b8[s] = *reinterpret_cast<const v4i *>(lds + j * TAIL_TILE + BM * kTileBytes +
                                                       swz(wn_e * WTN + fn * 32 + li_e, 2 * s + lh_e));
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    a8[s][fm] = *reinterpret_cast<const v4i *>(lds + j * TAIL_TILE +
                                                               swz(wm_e * WTM + fm * 32 + li_e, 2 * s + lh_e));
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if (j == 0 && s == 0)
                        mma_i8_0(acc8[fm], b8[s], a8[s][fm]);     // no VALU zero-fill to wait on
                    else
                        mma_i8(acc8[fm], b8[s], a8[s][fm]);
                }
        }
        // the column's scales (the same for its four blocks) and the rows'
        // scales, read while the tail MFMAs run
        float cs4[16], cs8[16], rs4[FM], rs8[FM];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 c4 = *reinterpret_cast<const float4 *>(sS + 2 * BM + nl + q * 8);
            const float4 c8 = *reinterpret_cast<const float4 *>(sS + 3 * BM + nl + q * 8);
            cs4[4 * q] = c4.x, cs4[4 * q + 1] = c4.y, cs4[4 * q + 2] = c4.z, cs4[4 * q + 3] = c4.w;
            // tail scales are not loaded when T8 == 0
            cs8[4 * q] = T8 > 0 ? c8.x : 0.0f, cs8[4 * q + 1] = T8 > 0 ? c8.y : 0.0f;
            cs8[4 * q + 2] = T8 > 0 ? c8.z : 0.0f, cs8[4 * q + 3] = T8 > 0 ? c8.w : 0.0f;
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int ml = wm_e * WTM + fm * 32 + li_e;
            rs4[fm] = sS[ml];
            rs8[fm] = T8 > 0 ? sS[BM + ml] : 0.0f;
        }
        // the tail sums come from MFMAs the compiler does not see as such:
        // their wait states before the VALU reads them
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int ml = wm_e * WTM + fm * 32 + li_e;
            const int m = row0 + ml;
            if constexpr (EXPORT) {
                // accumulator export (test path): this workgroup owns the sums
                if (m < a.M) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int n = col0 + nl + (r / 4) * 8 + (r % 4);
                        if (n < a.N) {
                            const int64_t e = (int64_t)m * a.N + n;
                            a.acc4_out[e] = (int32_t)acc[fm][fn][r];
                            if (a.acc8_out)
                                a.acc8_out[e] = acc8[fm][r];
                        }
                    }
                }
            }
            _Float16 *row = a.y + (int64_t)m * a.ldy + col0 + nl;
            // the block's head sums are read from the AGPRs here, not earlier
            asm volatile("" : "+a"(acc[fm][fn]));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = y_value(acc[fm][fn][q * 4 + e], acc8[fm][q * 4 + e], rs4[fm] * cs4[q * 4 + e],
                                   rs8[fm] * cs8[q * 4 + e]);
                const uint2 packed = uint2{pack_half2(v[0], v[1]), pack_half2(v[2], v[3])};
                if constexpr (INTERIOR) {
                    // The block goes through the wave's LDS slot (rows of
                    // Y_ROW bytes) so that Y is written as 64-byte row pieces,
                    // 16 bytes per lane, instead of 16-byte pieces of 32 rows.
                    // A wave's LDS operations run in issue order, so the next
                    // block's writes follow this block's reads.
                    unsigned char *slot = lds + Y_SLOTS + wave_e * (32 * Y_ROW);
                    *reinterpret_cast<uint2 *>(slot + li_e * Y_ROW + 8 * lh_e + 16 * q) = packed;
                    if (q == 3) {
                        const int pr = lane_e >> 2, pc = lane_e & 3;
                        uint4 piece[2];
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            piece[i] = *reinterpret_cast<const uint4 *>(slot + (pr + 16 * i) * Y_ROW + 16 * pc);
                        _Float16 *dst = a.y + (int64_t)(row0 + wm_e * WTM + fm * 32 + pr) * a.ldy + col0 + wn_e * WTN +
                                        fn * 32 + pc * 8;
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            *reinterpret_cast<uint4 *>(dst + (int64_t)(16 * i) * a.ldy) = piece[i];
                    }
                } else if (m < a.M) {
                    const int n = col0 + nl + q * 8;
                    if (vec_store && n + 3 < a.N) {
                        *reinterpret_cast<uint2 *>(row + q * 8) = packed;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < a.N)
                                row[q * 8 + e] = (_Float16)v[e];
                    }
                }
            }
        }
    }
    };
    if (interior)                                   // uniform
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

}  // namespace gemm_fp6_impl

using namespace gemm_fp6_impl;

int64_t u6_operand_bytes(int64_t rows, int64_t pitch4) { return (rows + 31) / 32 * (pitch4 / 32) * kU6Block; }

hipError_t launch_repack_u6(const uint8_t *q4, int64_t rows, int64_t pitch4, uint8_t *u6, hipStream_t stream) {
    const int64_t total = (rows + 31) / 32 * (pitch4 / 32) * 32;
    if (total <= 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(repack_u6_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q4, rows, pitch4, u6);
    return hipGetLastError();
}

bool gemm_fp6_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group) {
    (void)M;
    (void)N;
    return (group == 0 || (group == 128 && K_n % 128 == 0)) && K_n > 0 &&
           w4a4_pitch8_bytes(n_out) / kTileBytes <= MAX_TAIL_TILES;
}

const char *gemm_fp6_kernel_name(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group) {
    if (!gemm_fp6_fits(M, N, K_n, n_out, group))
        return nullptr;
    if (gemm_fp6_decode_fits(M, K_n, group))
        return gemm_fp6_decode_kernel_name(M);
    return group == 0 ? "gemm_fp6_big_kernel<false>" : "gemm_fp6_group_kernel<false>";
}

hipError_t launch_gemm_fp6(const Fp6GemmArgs &a, int32_t group, bool export_acc, hipStream_t stream) {
    if (gemm_fp6_decode_fits(a.M, a.K_n, group))
        return launch_gemm_fp6_decode(a, export_acc, stream);
    if (group == 128)
        return launch_gemm_fp6_group(a, export_acc, stream);
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (export_acc)
        hipLaunchKernelGGL(gemm_fp6_big_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_fp6_big_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a4
