// Device helpers shared by the GEMM translation units (not part of the C ABI).
#pragma once

#include "w4a4_internal.h"

namespace w4a4 {
namespace gemm_impl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTileBytes = 64;   // bytes of each row per K-tile: 128 INT4 or 64 INT8 channels

// Exact widening of packed two's complement nibbles to int8 lanes that hold
// 16 * q: the high nibbles stay in place, the low ones move up by 4 bits.
__device__ __forceinline__ uint32_t nib_hi(uint32_t p) { return p & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_lo(uint32_t p) { return (p << 4) & 0xF0F0F0F0u; }

// s_waitcnt immediate with only vmcnt constrained (gfx9 encoding).
constexpr int vmcnt_only(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate with only lgkmcnt constrained.
constexpr int lgkmcnt_only(int n) { return 0xF | (0x3 << 14) | (0x7 << 4) | ((n & 0xF) << 8); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Accumulator export (test path of every GEMM kernel): the exact integer
// partial sum a lane holds is added into the zeroed export array. Integer
// additions are exact and commute, so the parts of one scale group that
// different waves or workgroups hold give the same total in any order. The
// adds share vmcnt with the DMA, so a kernel waits for vmcnt(0) after them.
__device__ __forceinline__ void export_add(int32_t *dst, int v) { atomicAdd(dst, v); }

// Byte offset of 16-byte chunk c of row r inside a K-tile of 64-byte rows.
// Chunk c of row r is stored at slot (c ^ (r >> 1) ^ (r >> 2)) & 3: any 8
// consecutive rows then land on 8 distinct 16-byte slots modulo 128 bytes and
// any 16 on 16 distinct slots modulo 256 bytes, so a ds_read_b128 of 32 rows
// is free of bank conflicts whether the banks serve 8 or 16 lanes per pass.
__device__ __forceinline__ int swz(int r, int c) { return (r << 6) | (((c ^ (r >> 1) ^ (r >> 2)) & 3) << 4); }

// The DMA lane q of a tile (16 bytes) holds row r = q / 4 and global chunk
// ((q % 4) ^ (r >> 1) ^ (r >> 2)) & 3 of that row: the byte offset of that
// chunk inside the row's 64-byte segment.
__device__ __forceinline__ uint32_t dma_chunk_offset(int q) {
    const int r = q >> 2;
    return (uint32_t)((((q & 3) ^ (r >> 1) ^ (r >> 2)) & 3) * 16);
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 6 * per_tile]: the count must be
// an immediate, so the few values a ring can leave outstanding are spelled out.
template <int PER_TILE>
__device__ __forceinline__ void wait_tiles(int tiles_outstanding) {
    switch (tiles_outstanding) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_only(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_only(1 * PER_TILE)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * PER_TILE)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * PER_TILE)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_only(4 * PER_TILE)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_only(5 * PER_TILE)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_only(6 * PER_TILE)); break;
    }
}

// Output tile of a workgroup: consecutive workgroups are dealt round-robin
// to the 8 XCDs, so when the tile count is a multiple of 8 each XCD gets a
// contiguous range of tiles; tiles are then walked in bands of 8 tile rows
// (operand rows shared inside an XCD's L2).
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, bool xcd_remap, int &tm,
                                            int &tn) {
    const int tiles = tiles_m * tiles_n;
    if (xcd_remap && tiles % 8 == 0)
        tile = (tile % 8) * (tiles / 8) + tile / 8;
    constexpr int BAND = 8;
    const int band = tile / (BAND * tiles_n);
    const int first_m = band * BAND;
    const int band_m = min(tiles_m - first_m, BAND);
    const int in_band = tile - band * BAND * tiles_n;
    tm = first_m + in_band % band_m;
    tn = in_band / band_m;
}

}  // namespace gemm_impl
}  // namespace w4a4
