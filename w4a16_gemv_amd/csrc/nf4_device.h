// nf4_device.h -- device helpers shared by the libnf4 HIP sources (private).
//
// [blog] = the page "NF4反量化算子优化" (roundaboutt.github.io), whose "naive"
// section prints the NF4 table to 8 decimals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [p, p + bytes): loads beyond `bytes` return zeros and
// stores beyond it are dropped, so masked lanes need no branch (a branch
// around a load makes the compiler wait for every load in flight, including
// the prefetch of the next row group).
// A resource over a NULL pointer is always empty, so that a skipped matrix
// (whose descriptor is zeroed) can never be read or written.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           p ? static_cast<int>(bytes) : 0, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // beyond every resource (< 2^31 bytes)
constexpr uint32_t kFar = 0x40000000u;  // added to an in-range offset: still < 2^31, never wraps
// Cache-policy operand of the packed-weight loads: the nt (streaming) bit.
// Every weight byte is read once per launch, so there is nothing to keep.
constexpr int kStreamLoad = 2;

constexpr int kPairCopies = 32;

// The decode table: entry b = (hi, lo) where hi holds the bf16 pair
// (NF4[b >> 4], NF4[b & 15]) and lo the bf16 pair of the exact differences
// v - bf16(v), replicated kPairCopies times (copy c of entry b at uint2 index
// 32 b + c).  Each of the 256 entries is computed once by two threads, each
// of which writes 16 of its copies; the copy order is rotated by the entry,
// so the 64 lanes of a wave write 32 distinct bank pairs at a time.
__device__ __forceinline__ void build_pair_table(uint2* s_pairs, int tid, int nthreads) {
  static_assert(kPairCopies == 32, "two threads per entry, 16 copies each");
  for (int w = tid; w < 512; w += nthreads) {
    const int b = w & 255, half = w >> 8;
    const float ve = nf4_value(b >> 4), vo = nf4_value(b & 15);
    const uint32_t hi = pack_pair<NF4_BF16>(ve, vo);
    const float he = __builtin_bit_cast(float, hi << 16);
    const float ho = __builtin_bit_cast(float, hi & 0xFFFF0000u);
    const uint32_t lo2 = pack_pair<NF4_BF16>(ve - he, vo - ho);  // exact differences
    const uint2 entry = make_uint2(hi, lo2);
#pragma unroll
    for (int k = 0; k < 16; ++k) s_pairs[b * kPairCopies + ((b + 16 * half + k) & 31)] = entry;
  }
}



// --- host helpers ---

// Compute units of the current device, cached per device id.  The cache
// entries are atomics: threads that race on the first call of a device each
// query the attribute and store the same value.
inline int device_cus() {
  static std::atomic<int> cache[64];  // zero-initialized (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline nf4_status launch_status() {
  return hipGetLastError() == hipSuccess ? NF4_OK : NF4_EHIP;
}


}  // namespace nf4dev
