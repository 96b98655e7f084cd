// nf4_quantize.hip -- the NF4 encoders on the GPU: double-quantized, and the
// single-level format (one fp32 absmax per block, its level-1 step alone).
//
// Produces the format that nf4_dequant / nf4_gemv read, from fp32 weights,
// following the two levels described on the pages: [blog] "NF4反量化算子优化",
// section "双量化" (64-element blocks, absmax per block, nearest NF4 code, two
// codes per byte; block scales grouped by 256 and re-quantized), and [report]
// "NF4 双重量化反量化 CUDA Kernel 实现报告" §1.1-§1.2 (absmax_q uint8 index into
// code2 fp16[256], absmax2 fp16 per group, a global fp32 offset).
//
// Readings fixed here (the pages leave them open):
//  - level-1 codes are chosen against the true fp32 block absmax; a zero block
//    gets code 7 (the exact zero); ties go to the smaller code index;
//  - offset = mean of the block absmax values: one fp64 sum in block-index
//    order starting from +0, divided by the number of blocks and rounded once
//    to fp32;
//  - level 2 centres each block absmax by offset, absmax2 = fp16 (nearest) of
//    the group's largest |centred|, and absmax_q = the nearest code2 entry to
//    centred / absmax2 (0 when absmax2 is 0), all in fp32;
//  - code2 (linear variant) = the fp16 nearest to -1 + 2 i / 255.
// Every decision (max, divide, compare) is an exact or correctly rounded fp32
// operation, so the encoding is deterministic and independent of the launch.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "int4.h"
#include "nf4.h"
#include "nf4_device.h"

namespace {

using namespace nf4dev;

constexpr int kThreads = 256;
constexpr int kSumTile = 4096;  // block absmax values per LDS tile of the offset sum

uint32_t grid_for(int64_t items) {
  const int64_t g = (items + kThreads - 1) / kThreads;
  return static_cast<uint32_t>(g < 65536 ? g : 65536);
}

// absmax of each block of 2^log2bs consecutive elements (the last block may be
// short).
__global__ __launch_bounds__(kThreads) void block_absmax_kernel(const float* __restrict__ w,
                                                                 int64_t n, int log2bs,
                                                                 float* __restrict__ absmax) {
  const int64_t nb = ((n - 1) >> log2bs) + 1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb; b += stride) {
    const int64_t e0 = b << log2bs;
    const int64_t e1 = (b + 1) << log2bs < n ? (b + 1) << log2bs : n;
    float m = 0.0f;
    for (int64_t e = e0; e < e1; ++e) m = fmaxf(m, fabsf(w[e]));
    absmax[b] = m;
  }
}

// offset = fp32(fp64 sum of absmax[0..nb) in index order / nb).  The sum is
// one dependent chain of fp64 adds, so one thread does it; the workgroup
// streams the values into two LDS tiles so that the next tile's loads are in
// flight while thread 0 adds the current one.
__global__ __launch_bounds__(kThreads) void offset_kernel(const float* __restrict__ absmax,
                                                          int64_t nb, float* __restrict__ offset) {
  __shared__ float s_tile[2][kSumTile];
  const int t = threadIdx.x;
  const int64_t ntiles = (nb + kSumTile - 1) / kSumTile;
  constexpr int kPer = kSumTile / kThreads;  // values each thread stages per tile
  float v[kPer];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t b = tile * kSumTile + i * kThreads + t;
      v[i] = b < nb ? absmax[b] : 0.0f;
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) s_tile[buf][i * kThreads + t] = v[i];
  };
  fetch(0);
  put(0);
  __syncthreads();
  double sum = 0.0;
  for (int64_t c = 0; c < ntiles; ++c) {
    const bool more = c + 1 < ntiles;
    if (more) fetch(c + 1);  // in flight during the adds below
    if (t == 0) {
      const float* tile = s_tile[c & 1];
      const int64_t left = nb - c * kSumTile;
      const int cnt = left < kSumTile ? static_cast<int>(left) : kSumTile;
      for (int i = 0; i < cnt; ++i) sum += static_cast<double>(tile[i]);
    }
    if (more) put((c + 1) & 1);  // the other tile: thread 0 read it before the last barrier
    __syncthreads();
  }
  if (t == 0) offset[0] = static_cast<float>(sum / static_cast<double>(nb));
}

// absmax2[g] = fp16(max over the group's blocks of |absmax - offset|)
__global__ __launch_bounds__(kThreads) void group_scale_kernel(const float* __restrict__ absmax,
                                                                int64_t nb, int log2s2,
                                                                const float* __restrict__ offset,
                                                                uint16_t* __restrict__ absmax2) {
  const int64_t ng = ((nb - 1) >> log2s2) + 1;
  const float off = offset[0];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < ng; g += stride) {
    const int64_t b0 = g << log2s2;
    const int64_t b1 = (g + 1) << log2s2 < nb ? (g + 1) << log2s2 : nb;
    float m = 0.0f;
    for (int64_t b = b0; b < b1; ++b) m = fmaxf(m, fabsf(absmax[b] - off));
    absmax2[g] = to_half_bits<NF4_FP16>(m);
  }
}

// absmax_q[b] = index of the nearest code2 value to (absmax - offset) / absmax2
__global__ __launch_bounds__(kThreads) void block_code_kernel(const float* __restrict__ absmax,
                                                               int64_t nb, int log2s2,
                                                               const float* __restrict__ offset,
                                                               const uint16_t* __restrict__ absmax2,
                                                               const uint16_t* __restrict__ code2,
                                                               uint8_t* __restrict__ absmax_q) {
  __shared__ float s_code2[256];
  s_code2[threadIdx.x] = f16_to_f32(code2[threadIdx.x]);
  __syncthreads();
  const float off = offset[0];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb; b += stride) {
    const float a2 = f16_to_f32(absmax2[b >> log2s2]);
    const float c = absmax[b] - off;
    const float r = a2 == 0.0f ? 0.0f : c / a2;
    int best = 0;
    float bestd = fabsf(r - s_code2[0]);
    for (int i = 1; i < 256; ++i) {
      const float d = fabsf(r - s_code2[i]);
      if (d < bestd) {
        bestd = d;
        best = i;
      }
    }
    absmax_q[b] = static_cast<uint8_t>(best);
  }
}

__device__ __forceinline__ uint32_t nearest_nf4(float r, const float* s_nf4) {
  uint32_t best = 0;
  float bestd = fabsf(r - s_nf4[0]);
#pragma unroll
  for (int j = 1; j < 16; ++j) {
    const float d = fabsf(r - s_nf4[j]);
    if (d < bestd) {
      bestd = d;
      best = j;
    }
  }
  return best;
}

// two level-1 codes per byte, the even element in the high nibble
__global__ __launch_bounds__(kThreads) void pack_codes_kernel(const float* __restrict__ w,
                                                               int64_t n, int log2bs,
                                                               const float* __restrict__ absmax,
                                                               uint8_t* __restrict__ packed) {
  __shared__ float s_nf4[16];
  if (threadIdx.x < 16) s_nf4[threadIdx.x] = kNF4[threadIdx.x];
  __syncthreads();
  const int64_t nbytes = (n + 1) / 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < nbytes;
       i += stride) {
    uint32_t code[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t e = 2 * i + h;
      if (e >= n) continue;  // pad nibble of an odd-length tensor
      const float m = absmax[e >> log2bs];
      code[h] = m == 0.0f ? 7u : nearest_nf4(w[e] / m, s_nf4);
    }
    packed[i] = static_cast<uint8_t>((code[0] << 4) | code[1]);
  }
}

// The INT4 asymmetric group encoder ([handbook] "量化公式"): one thread per
// group of 2^lg elements (lg >= 1, so no byte is shared by two groups).
// Readings: s = fp16(fp32(max - min) / 15), replaced by 1 when it is 0;
// z = round(-min / s) with the stored s, kept as fp16; q = clamp(round(w / s)
// + z, 0, 15); round is to nearest, halves away from zero; the first element
// of each byte goes to the low nibble.
__global__ __launch_bounds__(kThreads) void int4_group_kernel(const float* __restrict__ w,
                                                               int64_t n, int lg,
                                                               uint8_t* __restrict__ packed,
                                                               uint16_t* __restrict__ scales,
                                                               uint16_t* __restrict__ zeros) {
  const int64_t ng = ((n - 1) >> lg) + 1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < ng;
       g += stride) {
    const int64_t e0 = g << lg;
    const int64_t e1 = (g + 1) << lg < n ? (g + 1) << lg : n;
    float mn = w[e0], mx = w[e0];
    for (int64_t e = e0 + 1; e < e1; ++e) {
      const float v = w[e];
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    const float range = mx - mn;
    uint16_t s16 = to_half_bits<NF4_FP16>(range / 15.0f);
    float s = f16_to_f32(s16);
    if (s == 0.0f) {
      s16 = 0x3C00u;  // 1.0
      s = 1.0f;
    }
    const uint16_t z16 = to_half_bits<NF4_FP16>(roundf(-mn / s));
    const float z = f16_to_f32(z16);
    scales[g] = s16;
    zeros[g] = z16;
    for (int64_t e = e0; e < e1; e += 2) {
      uint32_t code[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (e + h >= e1) continue;  // pad nibble of an odd-length tensor
        float q = roundf(w[e + h] / s) + z;
        q = q < 0.0f ? 0.0f : (q > 15.0f ? 15.0f : q);
        code[h] = static_cast<uint32_t>(q);
      }
      packed[e >> 1] = static_cast<uint8_t>(code[0] | (code[1] << 4));
    }
  }
}

bool pow2_log2(int32_t v, int* lg) {
  if (v < 1 || v > (1 << 30) || (v & (v - 1)) != 0) return false;
  int l = 0;
  while ((1 << l) < v) ++l;
  *lg = l;
  return true;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

extern "C" {

void nf4_code2_linear(uint16_t out[256]) {
  for (int i = 0; i < 256; ++i) {
    const _Float16 h = static_cast<_Float16>(-1.0 + 2.0 * static_cast<double>(i) / 255.0);
    out[i] = __builtin_bit_cast(uint16_t, h);
  }
}

size_t nf4_quantize_workspace_size(int64_t n, int32_t blocksize) {
  if (n <= 0 || blocksize < 1) return 0;
  const int64_t nb = (n + blocksize - 1) / blocksize;
  return align256(static_cast<size_t>(nb) * sizeof(float));
}

nf4_status nf4_quantize(const float* w, int64_t n, int32_t blocksize, int32_t s2_blocksize,
                        const uint16_t* code2, uint8_t* packed, uint8_t* absmax_q,
                        uint16_t* absmax2, float* offset, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int lbs = 0, ls2 = 0;
  if (n < 0 || !pow2_log2(blocksize, &lbs) || !pow2_log2(s2_blocksize, &ls2)) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!w || !code2 || !packed || !absmax_q || !absmax2 || !offset || !workspace)
    return NF4_EINVAL;
  if (n >= (int64_t(1) << 40)) return NF4_EUNSUPPORTED;
  if (workspace_bytes < nf4_quantize_workspace_size(n, blocksize)) return NF4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return NF4_EINVAL;
  const int64_t nb = (n + blocksize - 1) / blocksize;
  const int64_t ng = (nb + s2_blocksize - 1) / s2_blocksize;
  float* absmax = static_cast<float*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(block_absmax_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, st, w, n, lbs,
                     absmax);
  hipLaunchKernelGGL(offset_kernel, dim3(1), dim3(kThreads), 0, st, absmax, nb, offset);
  hipLaunchKernelGGL(group_scale_kernel, dim3(grid_for(ng)), dim3(kThreads), 0, st, absmax, nb,
                     ls2, offset, absmax2);
  hipLaunchKernelGGL(block_code_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, st, absmax, nb,
                     ls2, offset, absmax2, code2, absmax_q);
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for((n + 1) / 2)), dim3(kThreads), 0, st, w, n,
                     lbs, absmax, packed);
  return hipGetLastError() == hipSuccess ? NF4_OK : NF4_EHIP;
}

nf4_status nf4_quantize_absmax32(const float* w, int64_t n, int32_t blocksize, uint8_t* packed,
                                 float* absmax, void* stream) {
  int lbs = 0;
  if (n < 0 || !pow2_log2(blocksize, &lbs)) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!w || !packed || !absmax || (reinterpret_cast<uintptr_t>(absmax) & 3) != 0)
    return NF4_EINVAL;
  if (n >= (int64_t(1) << 40)) return NF4_EUNSUPPORTED;
  const int64_t nb = (n + blocksize - 1) / blocksize;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(block_absmax_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, st, w, n, lbs,
                     absmax);
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for((n + 1) / 2)), dim3(kThreads), 0, st, w, n,
                     lbs, absmax, packed);
  return hipGetLastError() == hipSuccess ? NF4_OK : NF4_EHIP;
}

nf4_status int4_quantize(const float* w, int64_t n, int32_t group_size, uint8_t* packed,
                         uint16_t* scales, uint16_t* zeros, void* stream) {
  int lg = 0;
  if (n < 0 || !pow2_log2(group_size, &lg) || lg < 1) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!w || !packed || !scales || !zeros) return NF4_EINVAL;
  if (n >= (int64_t(1) << 40)) return NF4_EUNSUPPORTED;
  const int64_t ng = ((n - 1) >> lg) + 1;
  hipLaunchKernelGGL(int4_group_kernel, dim3(grid_for(ng)), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), w, n, lg, packed, scales, zeros);
  return hipGetLastError() == hipSuccess ? NF4_OK : NF4_EHIP;
}

}  // extern "C"
