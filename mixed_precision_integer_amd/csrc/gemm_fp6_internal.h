// Internal declarations of the FP6 prefill GEMM (gemm_fp6.hip); not part of
// the public C ABI (include/w4a4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// Arguments of the FP6 GEMM. The INT4 head operands are in the u6 block
// layout (see gemm_fp6.hip).
struct Fp6GemmArgs {
    const uint8_t *a_u6;           // activations
    const uint8_t *w_u6;           // weights
    const int8_t *a8, *w8;         // INT8 tails [rows, pitch8]
    const float *sa4, *sa8, *sw4, *sw8;
    _Float16 *y;                   // [M, ldy]
    int32_t *acc4_out;             // [M, N] exact head sums (export) or nullptr
    int32_t *acc8_out;             // [M, N] or nullptr
    int32_t M, N, K_n, n_out;
    int64_t pitch4, pitch8, ldy;
};

// Bytes of a u6 operand, and the conversion of packed nibbles [rows, pitch4] to it.
int64_t u6_operand_bytes(int64_t rows, int64_t pitch4);
hipError_t launch_repack_u6(const uint8_t *q4, int64_t rows, int64_t pitch4, uint8_t *u6, hipStream_t stream);

// Shapes the FP6 GEMM takes, and the kernel it launches for them.
bool gemm_fp6_fits(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group);
const char *gemm_fp6_kernel_name(int32_t M, int32_t N, int32_t K_n, int32_t n_out, int32_t group);
hipError_t launch_gemm_fp6(const Fp6GemmArgs &a, int32_t group, bool export_acc, hipStream_t stream);
// The group-scale kernel (group 128; gemm_fp6_group.hip).
hipError_t launch_gemm_fp6_group(const Fp6GemmArgs &a, bool export_acc, hipStream_t stream);
// The decode kernel for 33..128 token rows with group 128 (gemm_fp6_decode.hip).
bool gemm_fp6_decode_fits(int32_t M, int32_t K_n, int32_t group);
const char *gemm_fp6_decode_kernel_name(int32_t M);
hipError_t launch_gemm_fp6_decode(const Fp6GemmArgs &a, bool export_acc, hipStream_t stream);

}  // namespace w4a4
