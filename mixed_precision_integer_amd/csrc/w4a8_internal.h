// Internal declarations of the W4A8 GEMM (gemm_w4a8.hip); not part of the
// public C ABI.
#pragma once

#include "w4a4_internal.h"

namespace w4a4 {

// INT8 activations a.a8 [M, pitch8] with token scales a.sa8 [M] times INT4
// weights a.w4 [N, pitch4] with scales a.sw4 [N, G]; K_n = K channels, a
// multiple of 128, group 0 or a multiple of 128. export_acc: write the exact
// group sums to a.acc4_out [G, M, N] instead of Y.
hipError_t launch_gemm_w4a8(const GemmArgs &a, bool export_acc, hipStream_t stream);

}  // namespace w4a4
