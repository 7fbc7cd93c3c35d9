// Internal declarations of the quantization-side kernels (row quantizer,
// outlier selection, KV cache) shared by their translation units and the C
// ABI. Nothing here is part of the public C ABI (include/w4a4.h); the GEMM
// declarations live in w4a4_internal.h.
#pragma once

#include "w4a4_internal.h"

namespace w4a4 {

// Arguments of the row quantizer: one launch quantizes `rows` rows of a
// [rows, ld] fp16 matrix (activations or weights).
struct QuantArgs {
    const _Float16 *src;
    int64_t ld;
    const int32_t *perm;
    int32_t rows, K, n_out, K_n, group, G;
    uint8_t *q4;          // [rows, pitch4] packed nibbles, or nullptr when u6 is set
    uint8_t *u6;          // the head as the FP6 GEMM's u6 operand instead of nibbles (group 0 only), or nullptr
    int8_t *q8;           // [rows, pitch8]
    float *s4;            // [rows, G]
    float *s8;            // [rows] or nullptr
    int64_t pitch4, pitch8;
    // RMSNorm in front of the quantizer (nullptr gamma: none)
    const _Float16 *gamma;  // [K] norm weight, original channel order
    float eps;
    float *rstd;          // [rows] norm factor per row, or nullptr
};

hipError_t launch_quant_rows(const QuantArgs &a, hipStream_t stream);
int quant_rows_max_k();   // longest row (channels) the quantizer takes

// Offline outlier-channel selection (select_kernels.hip).
struct SelectArgs {
    const void *X;        // [rows, ld] fp16 calibration batch
    int64_t ld;
    int32_t rows, K, n_out;
    int32_t *outlier_idx; // [n_out] or nullptr
    int32_t *perm;        // [K]
    void *absmax;         // [K] fp16 or nullptr
    void *workspace;      // plan_select(rows, K).workspace_bytes, 256-byte aligned
};

struct SelectPlan {
    int stripes, chunks, rows_per_chunk;
    int64_t kp;                   // channels rounded up to 8
    size_t keys_offset, workspace_bytes;
};

SelectPlan plan_select(int32_t rows, int32_t K);
int select_max_k();
hipError_t launch_select(const SelectArgs &a, hipStream_t stream);

// Low-bit KV cache (kv_kernels.hip): the key or value vectors of T tokens,
// X [T, ldx] fp16 with H heads of D channels each, quantized into slots of a
// cache of num_slots slots (codes [num_slots, H, D * bits / 8] bytes, scales
// [num_slots, H] fp32), or gathered back into Y [T, ldy] fp16.
struct KvArgs {
    const _Float16 *X;
    int64_t ldx;
    _Float16 *Y;
    int64_t ldy;
    int32_t T, H, D, bits;
    const int32_t *slots;  // [T] cache slot of each token, or nullptr (slot = token)
    int64_t num_slots;
    uint8_t *cq;
    float *cs;
};

hipError_t launch_kv(const KvArgs &a, bool quant, hipStream_t stream);

}  // namespace w4a4
