// Device-side pieces shared by the FP6 GEMM kernels (gemm_fp6.hip,
// gemm_fp6_group.hip): the u6 block size, the operand fragment read and the
// fp16 packing of results.
#pragma once

#include "gemm_common.h"

namespace w4a4 {
namespace gemm_fp6_impl {

using namespace gemm_impl;

constexpr int64_t kU6Block = 1536;                 // bytes of a 32-row x 64-channel u6 block
constexpr int BLK = (int)kU6Block;                 // one 32-row block of a K-tile (64 channels)
constexpr int MAX_TAIL_TILES = 4;                  // INT8 tail <= 256 channels

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

// One operand fragment: 64 FP6 values of one row, as six dwords (the
// 16-byte lo part of the chunk image, then its 8-byte hi part). The FP6
// matrix instruction reads only these six registers of an operand.
__device__ __forceinline__ v6i load_operand(const unsigned char *lo, const unsigned char *hi) {
    const v4i l = *reinterpret_cast<const v4i *>(lo);
    const v2i h = *reinterpret_cast<const v2i *>(hi);
    v6i v;
    v.s0123 = l;
    v.s45 = h;
    return v;
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    const _Float16 l = (_Float16)lo, h = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

}  // namespace gemm_fp6_impl
}  // namespace w4a4
