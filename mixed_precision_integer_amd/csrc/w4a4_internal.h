// Internal declarations shared by the HIP translation units of libw4a4.
// Nothing here is part of the public C ABI (include/w4a4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// Arguments of the row quantizer: one launch quantizes `rows` rows of a
// [rows, ld] fp16 matrix (activations or weights).
struct QuantArgs {
    const _Float16 *src;
    int64_t ld;
    const int32_t *perm;
    int32_t rows, K, n_out, K_n, group, G;
    uint8_t *q4;          // [rows, pitch4]
    int8_t *q8;           // [rows, pitch8]
    float *s4;            // [rows, G]
    float *s8;            // [rows] or nullptr
    int64_t pitch4, pitch8;
};

hipError_t launch_quant_rows(const QuantArgs &a, hipStream_t stream);

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
};

hipError_t launch_gemm(const GemmArgs &a, bool export_acc, hipStream_t stream);

}  // namespace w4a4
