// Shared pieces of the attention kernels (bf16 MFMA operand types, packing helpers).
#pragma once

#include "common.h"

namespace specv {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTileKeys = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // round-to-nearest-even fp32 -> bf16, two values per word (one v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

}  // namespace attn
}  // namespace specv
