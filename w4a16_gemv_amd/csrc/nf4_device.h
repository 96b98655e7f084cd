// nf4_device.h -- device helpers shared by the libnf4 HIP sources (private).
//
// [blog] = the page "NF4反量化算子优化" (roundaboutt.github.io), whose "naive"
// section prints the NF4 table to 8 decimals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4.h"

namespace nf4dev {

// The 16 NF4 code values, as the 8-decimal literals printed in [blog] "naive";
// each literal is rounded to the nearest fp32 by the compiler.
__device__ constexpr float kNF4[16] = {
    -1.00000000f, -0.69619280f, -0.52507305f, -0.39491749f,
    -0.28444138f, -0.18477343f, -0.09105004f, 0.00000000f,
    0.07958030f,  0.16093020f,  0.24611230f,  0.33791524f,
    0.44070983f,  0.56261700f,  0.72295684f,  1.00000000f,
};

// NF4[i] for a runtime index without a memory access: a chain of selects over
// the literals (constant indices fold to immediates).
__device__ __forceinline__ float nf4_value(uint32_t i) {
  float v = kNF4[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) v = i == static_cast<uint32_t>(j) ? kNF4[j] : v;
  return v;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));  // exact widening
}

// Pin a value as an fp32 register.  Without it the compiler may fold an fp32
// multiply and the following 16-bit conversion into one mixed-precision fma
// (v_fma_mixlo_f16), which rounds the exact product straight to fp16 and skips
// the fp32 rounding the method prescribes (a double-rounding difference).
__device__ __forceinline__ float as_fp32(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Two 16-bit outputs in one dword: the even element in the low half (lower
// address), the odd element in the high half.  Both inputs are first pinned as
// rounded fp32 values.
template <int OUT>
__device__ __forceinline__ uint32_t pack_pair(float even, float odd) {
  even = as_fp32(even);
  odd = as_fp32(odd);
  if constexpr (OUT == NF4_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){even, odd}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){even, odd}, f16x2));
  }
}

template <int OUT>
__device__ __forceinline__ uint16_t to_half_bits(float v) {
  return static_cast<uint16_t>(pack_pair<OUT>(v, 0.0f) & 0xFFFFu);
}

}  // namespace nf4dev
