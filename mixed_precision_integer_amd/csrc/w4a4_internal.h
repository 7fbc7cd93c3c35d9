// Internal declarations shared by the HIP translation units of libw4a4.
// Nothing here is part of the public C ABI (include/w4a4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a4 {

// Direct global->LDS DMA (gfx950 global_load_lds): lane i's bytes land at
// M0 + i * size. Issued through inline asm so that the compiler does not put
// a wait for every outstanding DMA in front of each later LDS read; the
// kernels order DMA and LDS reads themselves with explicit vmcnt waits and
// workgroup barriers. The instructions return nothing to VGPRs.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// 16 bytes per lane from base + voff. base and lds are wave-uniform; they are
// moved to SGPRs explicitly (readfirstlane of a uniform value is exact).
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(sl)
                 : "memory", "m0");
}
// 4 bytes per lane from base + voff (base wave-uniform).
__device__ __forceinline__ void dma4s(const void *base, uint32_t voff, uint32_t lds) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sb), "s"(sl)
                 : "memory", "m0");
}
// The compiler waits for outstanding vector memory operations before it
// rewrites a register that one of these asm statements read, so the offset
// and address operands passed to them should stay in registers that are not
// recomputed inside a pipelined loop.
// 4 bytes per lane from a per-lane address
__device__ __forceinline__ void dma4(const void *p, uint32_t lds) {
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(p), "s"(sl) : "memory", "m0");
}

// Arguments of the mixed-precision GEMM.
struct GemmArgs {
    const uint8_t *a4;    // [M, pitch4] packed INT4 activations
    const int8_t *a8;     // [M, pitch8] INT8 outlier activations
    const uint8_t *w4;    // [N, pitch4]
    const int8_t *w8;     // [N, pitch8]
    const float *sa4, *sa8, *sw4, *sw8;
    _Float16 *y;          // [M, ldy]
    int32_t *acc4_out;    // [G, M, N] (accumulator export) or nullptr
    int32_t *acc8_out;    // [M, N] or nullptr
    int32_t M, N, K_n, n_out, group, G;
    int64_t pitch4, pitch8, ldy;
    int32_t splits;       // K splits (1: no split); set by launch_gemm
    float *part;          // [splits, M, N] fp32 partial sums (splits > 1)
    uint32_t *ctr;        // [output tiles] arrival counters, zero between calls
};

// Launch shape of the GEMM for one problem: a pure function of the shape.
struct GemmPlan {
    int cfg;                  // tile configuration: 0 64 x 64, 1 128 x 128, 2 256 x 256,
                              // 3 128 x 128 for 128-channel scale groups,
                              // 4 decode (M <= 128, weights streamed once)
    int tiles;                // output tiles
    int splits;               // K splits per output tile
    int mb;                   // decode: 32-row token blocks (1: gemm_decode_kernel)
    int rows;                 // decode: token rows
    size_t part_offset;       // byte offset of the fp32 partial sums (counters first)
    size_t part_bytes;        // fp32 partial sums
    size_t workspace_bytes;   // 0 when splits == 1
};

GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group);

// Bytes of the arrival-counter block at the start of every split-K workspace,
// and a kernel that zeroes that block on a stream (no memset node).
size_t gemm_counter_bytes();
hipError_t clear_gemm_counters(void *workspace, hipStream_t stream);

// Kernel of a plan, as named in a kernel trace (static string).
const char *gemm_kernel_name(const GemmPlan &p);

// `workspace` holds plan_gemm(...).workspace_bytes bytes; its counter part
// must be zero on entry and is zero again when the kernel completes. With
// export_acc the same kernel also adds its exact integer sums into
// a.acc4_out / a.acc8_out, which this call zeroes first.
hipError_t launch_gemm(const GemmArgs &a, bool export_acc, void *workspace, hipStream_t stream);

// Decode kernels for M <= 128 token rows (gemm_decode.hip).
bool gemm_decode_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group);
const char *decode_kernel_name(int rows);
hipError_t launch_gemm_decode(const GemmArgs &a, bool export_acc, hipStream_t stream);

// Decode layer call with the quantizer fused in (gemm_decode_fused.hip): at
// most 2 token rows, 128-channel groups, at most 128 outlier channels.
struct DecodeFusedArgs {
    const uint16_t *x;    // [M, ldx] fp16 activations (bit patterns)
    const uint16_t *gamma;  // [K] fp16 RMSNorm weights in front of the layer, or nullptr
    float eps;            // RMSNorm epsilon (with gamma)
    const int32_t *perm;  // [K] reordered channel -> source channel
    const uint8_t *w4;    // [N, pitch4]
    const int8_t *w8;     // [N, pitch8]
    const float *sw4, *sw8;
    _Float16 *y;          // [M, ldy]
    int32_t M, N, K, K_n, n_out;
    int64_t ldx, pitch4, pitch8, ldy;
};
bool decode_fused_fits(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group);
hipError_t launch_decode_fused(const DecodeFusedArgs &a, hipStream_t stream);

// 128 x 128 tile kernel for 128-channel scale groups (gemm_group.hip).
bool gemm_group_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group);
hipError_t launch_gemm_group(const GemmArgs &a, bool export_acc, hipStream_t stream);

// 256 x 256 tile kernel for one scale group per row (gemm_big.hip).
bool gemm_big_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t G);
hipError_t launch_gemm_big(const GemmArgs &a, bool export_acc, hipStream_t stream);

}  // namespace w4a4
