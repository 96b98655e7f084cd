// nf4_probe.hip -- bandwidth probes (measurement helpers): the hot path's
// memory streams without its arithmetic, to give its achieved bandwidth a
// measured ceiling on the same GPU.  See include/nf4_probe.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4.h"
#include "nf4_device.h"
#include "nf4_probe.h"

namespace {

using namespace nf4dev;

constexpr int kProbeThreads = 512;

// One contiguous range of 16-byte units per wave, four loads in flight per
// lane, streaming (non-temporal) like the GEMV's weight loads.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / 64);
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t per = (n16 + waves - 1) / waves;
  const int64_t beg = w * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  for (int64_t i = beg + lane; i < end; i += 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = i + 64 * u < end ? __builtin_nontemporal_load(src + i + 64 * u) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// The dequant's pattern: a workgroup owns 256 x 4 consecutive dwords, each
// lane takes 4 of them at a stride of 256 (coalesced loads), and writes 16
// bytes per dword with streaming stores.
__global__ __launch_bounds__(256) void probe_expand_kernel(const uint32_t* __restrict__ src,
                                                           int64_t n4, u32x4* __restrict__ dst) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x;
  uint32_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = base + 256 * u < n4 ? src[base + 256 * u] : 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + 256 * u < n4)
      __builtin_nontemporal_store(u32x4{v[u], v[u] ^ 1u, v[u] ^ 2u, v[u] ^ 3u}, dst + base + 256 * u);
}

}  // namespace

extern "C" {

nf4_status nf4_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return NF4_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0) return NF4_EINVAL;
  const int64_t cus = device_cus();
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<uint32_t>(cus * 2)), dim3(kProbeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<int64_t>(bytes / 16), sink);
  return launch_status();
}

nf4_status nf4_probe_expand_copy(const void* src, size_t src_bytes, void* dst, void* stream) {
  if (src_bytes == 0) return NF4_OK;
  if (!src || !dst || !aligned(src, 4) || !aligned(dst, 16) || src_bytes % 4 != 0) return NF4_EINVAL;
  const int64_t n4 = static_cast<int64_t>(src_bytes / 4);
  const int64_t blocks = (n4 + 1023) / 1024;
  if (blocks > 0x7FFFFFFF) return NF4_EUNSUPPORTED;
  hipLaunchKernelGGL(probe_expand_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint32_t*>(src), n4,
                     static_cast<u32x4*>(dst));
  return launch_status();
}

}  // extern "C"
