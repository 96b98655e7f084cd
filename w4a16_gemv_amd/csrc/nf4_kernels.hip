// nf4_kernels.hip -- gfx950 kernels and the C ABI of libnf4.
//
// NF4 double-quantization dequant ([report] §1.3) and the fused W4A16
// dequant-GEMV ([quanttax] "Kernel 实现"; [handbook] "GEMV kernel 的写法"),
// written for CDNA4: wave64, LDS-resident NF4 table, shift-based block/group
// indexing, one absmax_real per 64-element block, packed 128-bit stores,
// DPP wave reductions.  No MFMA: at batch <= 8 the GEMV is bound by HBM
// (batch 1) or by vector ALU issue (batch 4-8), not by a dense contraction.
//
// Pages (by title): [blog] "NF4反量化算子优化"; [report] "NF4 双重量化反量化
// CUDA Kernel 实现报告"; [quanttax] "RTX 4060 上的 LLM 量化实测";
// [handbook] "量化与 GEMV".
//
// Numerics.  This file is compiled with -ffp-contract=off: every product and
// sum of the dequant formula is rounded to fp32 on its own.  GEMV products are
// accumulated with explicit fmaf (fp32).  16-bit outputs use the gfx950 packed
// conversions v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32, which round to nearest
// even under the default rounding mode.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "int4.h"
#include "nf4.h"
#include "nf4_device.h"
#include "nf4_gemm.h"

namespace {

using namespace nf4dev;

// Where a block's scale comes from (a template parameter of every kernel).
// kFmtDouble: the double-quantized format, absmax_real = fp32(code2[absmax_q
// [block]] * absmax2[group]) + offset.  kFmtAbsmax32: one fp32 absmax per
// block and no second level; the absmax_q argument then carries that fp32
// array and absmax2, code2 and offset are not used.
// kFmtInt4: the INT4 asymmetric group format ([handbook] "量化公式", "W4A16：
// 在寄存器里反量化"): codes q in 0..15 with the FIRST element of each byte in
// the LOW nibble, and per group of 2^log2bs consecutive elements an fp16
// scale s (passed as absmax_q) and an fp16 zero point z (passed as absmax2):
// value = fp32(fp32(q - z) * s).
constexpr int kFmtDouble = 0;
constexpr int kFmtAbsmax32 = 1;
constexpr int kFmtInt4 = 2;

// Register type of a block's scale bits as loaded: the absmax_q byte, the
// fp32 absmax, or the fp16 group scale.
template <int FMT>
struct ScaleBits { using type = uint8_t; };
template <>
struct ScaleBits<kFmtAbsmax32> { using type = uint32_t; };
template <>
struct ScaleBits<kFmtInt4> { using type = uint16_t; };

// The code of element 2 i + odd in packed byte i: the high nibble holds the
// even element in the NF4 formats, the low nibble in the INT4 format.
template <int FMT>
__device__ __forceinline__ uint32_t nibble_of(uint32_t byte, uint32_t odd) {
  if constexpr (FMT == kFmtInt4)
    return odd ? (byte >> 4) & 15u : byte & 15u;
  else
    return odd ? byte & 15u : (byte >> 4) & 15u;
}

// absmax_real of one first-level block: fp32 product, then fp32 sum (or the
// stored fp32 absmax).
template <int FMT>
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ absmax_q,
                                             const uint16_t* __restrict__ absmax2,
                                             const uint16_t* __restrict__ code2, float offset,
                                             int64_t blk, int log2s2) {
  if constexpr (FMT == kFmtAbsmax32) {
    return reinterpret_cast<const float*>(absmax_q)[blk];
  } else {
    const float c = f16_to_f32(code2[absmax_q[blk]]);
    const float g = f16_to_f32(absmax2[blk >> log2s2]);
    const float s = c * g;
    return s + offset;
  }
}

// The value of one element with code `nib` in block (group) blk; tab holds
// the 16 NF4 values (the 16 integers 0..15 in the INT4 format).
template <int FMT>
__device__ __forceinline__ float element_value(const float* tab, uint32_t nib,
                                               const uint8_t* __restrict__ absmax_q,
                                               const uint16_t* __restrict__ absmax2,
                                               const uint16_t* __restrict__ code2, float offset,
                                               int64_t blk, int log2s2) {
  if constexpr (FMT == kFmtInt4) {
    const float s = f16_to_f32(reinterpret_cast<const uint16_t*>(absmax_q)[blk]);
    const float z = f16_to_f32(absmax2[blk]);
    const float d = tab[nib] - z;  // exact
    return d * s;
  } else {
    return tab[nib] * block_scale<FMT>(absmax_q, absmax2, code2, offset, blk, log2s2);
  }
}

// The table of the 16 code values: NF4, or the integers 0..15.
template <int FMT>
__device__ __forceinline__ float code_value(uint32_t i) {
  if constexpr (FMT == kFmtInt4)
    return static_cast<float>(i);
  else
    return nf4_value(i);
}

// ---------------------------------------------------------------------------
// Dequant, vectorized path.
//
// A workgroup of 256 lanes owns a tile of 256*U "steps"; a step is one packed
// dword (8 elements) in, one 16-byte store out.  Lane t handles steps
// tile0 + u*256 + t, so every wave-wide load covers 256 contiguous bytes and
// every wave-wide store 1 KiB of contiguous output.
//
// Every global load of the tile is issued before the first wait: the packed
// dwords, the tile's absmax_q bytes and absmax2 halves, and the 256-entry
// code2 table (staged in LDS as fp32, so that the code2[absmax_q] lookup is an
// LDS read instead of a second, dependent global load).  The workgroup then
// computes one absmax_real per first-level block into LDS (a 64-element block
// is shared by 8 lanes) and decodes with the NF4 table in LDS (lanes index it
// divergently; 16 distinct words never conflict on LDS banks).
// The output, four times the bytes of the input, goes out with streaming
// (non-temporal) stores.  Tiles are small (U = 4, fewer on inputs that would
// not give every CU a tile) so that several workgroups per CU sit at
// different phases and one's stores overlap another's loads.
// Requirements (checked on the host): packed 4-byte aligned, out 16-byte
// aligned, blocksize >= 8 so that a step never straddles a block.
// ---------------------------------------------------------------------------
constexpr int kDqThreads = 256;

template <int OUT, int U, int FMT = kFmtDouble>
__global__ __launch_bounds__(kDqThreads) void dequant_vec_kernel(
    const uint32_t* __restrict__ packed32, const uint8_t* __restrict__ packed8,
    const uint8_t* __restrict__ absmax_q, const uint16_t* __restrict__ absmax2,
    const uint16_t* __restrict__ code2, float offset, int64_t n, int log2bs, int log2s2,
    u32x4* __restrict__ out16, uint16_t* __restrict__ out2) {
  __shared__ float s_nf4[16];
  __shared__ float s_code2[256];
  __shared__ float s_scale[kDqThreads * U];
  __shared__ float s_zero[FMT == kFmtInt4 ? kDqThreads * U : 1];
  const int t = threadIdx.x;
  const int64_t full_steps = n >> 3;
  const int64_t step0 = static_cast<int64_t>(blockIdx.x) * (kDqThreads * U);

  // 1. all global loads of the tile, issued back to back
  uint32_t w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = step0 + u * kDqThreads + t;
    w[u] = s < full_steps ? packed32[s] : 0u;
  }
  const uint16_t c2 = FMT == kFmtDouble ? code2[t] : uint16_t(0);
  const int64_t e_begin = step0 * 8;
  const int64_t e_end = (step0 + kDqThreads * U) * 8 < n ? (step0 + kDqThreads * U) * 8 : n;
  const int64_t blk0 = e_begin >> log2bs;
  const int nblk = static_cast<int>(((e_end - 1) >> log2bs) - blk0 + 1);  // <= 256 * U
  uint32_t qv[U];
  uint16_t gv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = t + u * kDqThreads;
    if constexpr (FMT == kFmtAbsmax32) {
      qv[u] = i < nblk ? reinterpret_cast<const uint32_t*>(absmax_q)[blk0 + i] : 0u;
    } else if constexpr (FMT == kFmtInt4) {
      qv[u] = i < nblk ? reinterpret_cast<const uint16_t*>(absmax_q)[blk0 + i] : 0u;
      gv[u] = i < nblk ? absmax2[blk0 + i] : uint16_t(0);
    } else {
      qv[u] = i < nblk ? absmax_q[blk0 + i] : 0u;
      gv[u] = i < nblk ? absmax2[(blk0 + i) >> log2s2] : uint16_t(0);
    }
  }

  // 2. tables, then one absmax_real per block
  if constexpr (FMT == kFmtDouble) s_code2[t] = f16_to_f32(c2);
  if (t < 16) s_nf4[t] = code_value<FMT>(static_cast<uint32_t>(t));
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = t + u * kDqThreads;
    if (i < nblk) {
      if constexpr (FMT == kFmtAbsmax32) {
        s_scale[i] = __builtin_bit_cast(float, qv[u]);
      } else if constexpr (FMT == kFmtInt4) {
        s_scale[i] = f16_to_f32(static_cast<uint16_t>(qv[u]));
        s_zero[i] = f16_to_f32(gv[u]);
      } else {
        const float prod = s_code2[qv[u]] * f16_to_f32(gv[u]);
        s_scale[i] = prod + offset;
      }
    }
  }
  __syncthreads();

  // 3. decode 8 nibbles per step and store 16 bytes
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = step0 + u * kDqThreads + t;
    if (s < full_steps) {
      const int bi = static_cast<int>(((s * 8) >> log2bs) - blk0);
      const float a = s_scale[bi];
      const uint32_t wd = w[u];
      uint32_t o[4];
      if constexpr (FMT == kFmtInt4) {
        const float z = s_zero[bi];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float de = s_nf4[(wd >> (8 * j)) & 15u] - z;  // exact
          const float dd = s_nf4[(wd >> (8 * j + 4)) & 15u] - z;
          o[j] = pack_pair<OUT>(de * a, dd * a);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float ve = s_nf4[(wd >> (8 * j + 4)) & 15u] * a;
          const float vo = s_nf4[(wd >> (8 * j)) & 15u] * a;
          o[j] = pack_pair<OUT>(ve, vo);
        }
      }
      // streaming store: the kernel never reads its output back
      const u32x4 v = {o[0], o[1], o[2], o[3]};
      __builtin_nontemporal_store(v, out16 + s);
    } else if (s == full_steps) {
      // ragged tail: the last n % 8 elements, one at a time
      for (int64_t e = s * 8; e < n; ++e) {
        const uint32_t nib = nibble_of<FMT>(packed8[e >> 1], static_cast<uint32_t>(e & 1));
        const int bi = static_cast<int>((e >> log2bs) - blk0);
        const float a = s_scale[bi];
        if constexpr (FMT == kFmtInt4) {
          const float d = s_nf4[nib] - s_zero[bi];
          out2[e] = to_half_bits<OUT>(d * a);
        } else {
          out2[e] = to_half_bits<OUT>(s_nf4[nib] * a);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dequant, general path: one element per lane, byte loads, 16-bit stores.
// Used for unaligned buffers and block sizes below 8.  Same arithmetic, same
// bits.
// ---------------------------------------------------------------------------
template <int OUT, int FMT = kFmtDouble>
__global__ __launch_bounds__(256) void dequant_any_kernel(
    const uint8_t* __restrict__ packed8, const uint8_t* __restrict__ absmax_q,
    const uint16_t* __restrict__ absmax2, const uint16_t* __restrict__ code2, float offset,
    int64_t n, int log2bs, int log2s2, uint16_t* __restrict__ out2) {
  __shared__ float s_nf4[16];
  if (threadIdx.x < 16) s_nf4[threadIdx.x] = code_value<FMT>(threadIdx.x);
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += stride) {
    const uint32_t nib = nibble_of<FMT>(packed8[e >> 1], static_cast<uint32_t>(e & 1));
    out2[e] = to_half_bits<OUT>(
        element_value<FMT>(s_nf4, nib, absmax_q, absmax2, code2, offset, e >> log2bs, log2s2));
  }
}

// ---------------------------------------------------------------------------
// Wave64 sum with DPP: after the six steps lane 63 holds the total.
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror and
// row_mirror each row of 16, row_bcast:15 / row_bcast:31 carry row sums up.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int src = __builtin_bit_cast(int, v);
  const int moved = __builtin_amdgcn_update_dpp(0, src, CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sums of two per-lane values p and q over the 64 lanes at once: afterwards
// lanes 0-15 hold sum(p) and lanes 32-47 hold sum(q).  v_permlane32_swap
// pairs lane l with lane l + 32 (p in the low half, q in the high half),
// v_permlane16_swap against zero then folds rows 1 and 3 into rows 0 and 2,
// and four in-row DPP steps finish each row: 8 instructions for both sums,
// and no row broadcasts.
__device__ __forceinline__ float wave_sum_pair(float p, float q) {
  // (vector elements are copied to scalars before any bit_cast: a bit_cast
  // of a vector-element lvalue reads element 0 whatever the index)
  const auto h = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, p),
                                                  __builtin_bit_cast(uint32_t, q), false, false);
  const uint32_t h0 = h[0], h1 = h[1];
  const float s = __builtin_bit_cast(float, h0) + __builtin_bit_cast(float, h1);
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, s), 0u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  float t = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  t = dpp_add<0xB1, 0xF>(t);   // quad_perm [1,0,3,2]
  t = dpp_add<0x4E, 0xF>(t);   // quad_perm [2,3,0,1]
  t = dpp_add<0x141, 0xF>(t);  // row_half_mirror
  t = dpp_add<0x140, 0xF>(t);  // row_mirror
  return t;
}

// Sums of four per-lane values a, b, c, d over the 64 lanes at once:
// afterwards every lane of row 0 (lanes 0-15) holds sum(a), row 1 sum(c),
// row 2 sum(b) and row 3 sum(d).  Two v_permlane32_swap fold the wave halves
// (a and c into lanes 0-31, b and d into lanes 32-63), one v_permlane16_swap
// folds rows 1 and 3 into rows 0 and 2 while moving c and d to rows 1 and 3,
// and four in-row DPP steps finish: 10 instructions for the four sums.
__device__ __forceinline__ float wave_sum_quad(float a, float b, float c, float d) {
  const auto hab = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
  const auto hcd = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, c),
                                                    __builtin_bit_cast(uint32_t, d), false, false);
  const uint32_t ab0 = hab[0], ab1 = hab[1], cd0 = hcd[0], cd1 = hcd[1];
  const float sab = __builtin_bit_cast(float, ab0) + __builtin_bit_cast(float, ab1);
  const float scd = __builtin_bit_cast(float, cd0) + __builtin_bit_cast(float, cd1);
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, sab),
                                                  __builtin_bit_cast(uint32_t, scd), false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  float t = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  t = dpp_add<0xB1, 0xF>(t);   // quad_perm [1,0,3,2]
  t = dpp_add<0x4E, 0xF>(t);   // quad_perm [2,3,0,1]
  t = dpp_add<0x141, 0xF>(t);  // row_half_mirror
  t = dpp_add<0x140, 0xF>(t);  // row_mirror
  return t;
}

__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// ---------------------------------------------------------------------------
// Fused dequant-GEMV, streaming path (batch 1-2).
//
// Decode table.  One packed byte holds two weights, so the workgroup builds in
// LDS a 256-entry table: entry b = (NF4[b >> 4], NF4[b & 15]) as two fp32 (the
// even element first).  The table is replicated 32 times with copy c of entry
// b at byte address 256 b + 8 c; lane l reads copy l % 32, so the 32 lanes
// that LDS serves together always hit distinct bank pairs whatever bytes they
// hold (a single copy loses about half the LDS throughput to bank conflicts).
// The address of byte i of a packed dword d is then one v_perm_b32: byte i of
// d becomes address bits 8..15 and the lane's copy offset bits 0..7.  Per
// weight: half a VALU op of addressing, half a 64-bit LDS read, one fma.
//
// Work split.  A workgroup has T teams of nw waves, nw = ceil(K / 2048): wave
// s of a team owns the 32-column chunks [2048 s + 32 l, +32) (lane l) for the
// whole kernel and keeps their activations in registers as fp32.  Each team
// walks groups of R consecutive rows (grid-stride); for each row a lane reads
// one 16-byte packed chunk, which lies inside one first-level block
// (blocksize >= 32, K % 32 == 0), so its absmax_real is applied once, after
// the lane's 32 products are summed (scale after accumulate).  The loads of
// the team's next row group are issued before the current group is computed.
// Lane partials are summed with DPP and a team's wave partials through LDS in
// a fixed order (one barrier per group, double-buffered): deterministic.
// Requirements (checked on the host): K % 32 == 0, K <= 16384, blocksize >=
// 32, packed and x 16-byte aligned, blockDim = 64 * nw * T <= 512.
// ---------------------------------------------------------------------------
constexpr int kSlab = 2048;

constexpr int kMaxDescs = 1024;  // matrices per grouped launch

// The INT4 decode table (same 64 KiB of LDS): entry b is the exact bf16 pair
// (b & 15, b >> 4) -- the even element, in the low nibble, in the low half --
// replicated 64 times, copy c of entry b at uint32 index 64 b + c, so lane l
// reads copy l and the 64 lanes of a wave never share a bank.
constexpr int kInt4Copies = 64;
__device__ __forceinline__ void build_int4_table(uint32_t* tab, int tid, int nthreads) {
  for (int w = tid; w < 256 * kInt4Copies; w += nthreads) {
    const uint32_t b = static_cast<uint32_t>(w) / kInt4Copies;
    tab[w] = pack_pair<NF4_BF16>(static_cast<float>(b & 15u), static_cast<float>(b >> 4));
  }
}

// Decode table and lane copy offset of the format (LDS byte offset of the
// lane's copy within an entry row of 256 bytes).
template <int FMT>
__device__ __forceinline__ uint32_t build_decode_table(uint2* s_pairs, int tid, int nthreads,
                                                       int lane) {
  if constexpr (FMT == kFmtInt4) {
    build_int4_table(reinterpret_cast<uint32_t*>(s_pairs), tid, nthreads);
    return static_cast<uint32_t>(lane % kInt4Copies) * 4u;
  } else {
    build_pair_table(s_pairs, tid, nthreads);
    return static_cast<uint32_t>(lane % kPairCopies) * 8u;
  }
}

// Sum of the lane's activations of one batch row (raw bf16 pairs in x): the
// zero-point term of the INT4 format is z times this sum.
template <int N>
__device__ __forceinline__ float pair_sum(const uint32_t (&x)[N]) {
  typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
  const bf16x2_ one = __builtin_bit_cast(bf16x2_, 0x3F803F80u);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_, x[i]), one, acc, false);
  return acc;
}


// Buffer resources a team needs to load row groups of one matrix.
struct LoadBufs {
  __amdgpu_buffer_rsrc_t packed, absmax_q, absmax2;
};

// What a team needs to finish a row group of one matrix: where y goes, N and
// the matrix's offset.
struct OutBufs {
  __amdgpu_buffer_rsrc_t y;
  int N;
  float offset;
};

template <int FMT>
__device__ __forceinline__ LoadBufs load_bufs(const nf4_gemv_desc& d, int K, int log2bs,
                                              int log2s2) {
  LoadBufs lb;
  const uint64_t n = d.N > 0 ? static_cast<uint64_t>(d.N) * static_cast<uint64_t>(K) : 0;
  const uint64_t nb = n ? ((n - 1) >> log2bs) + 1 : 0;
  const uint64_t ng = nb ? ((nb - 1) >> log2s2) + 1 : 0;
  lb.packed = rsrc(d.packed, static_cast<uint32_t>(n >> 1));
  if constexpr (FMT == kFmtAbsmax32) {
    lb.absmax_q = rsrc(d.absmax_q, static_cast<uint32_t>(nb * 4));  // the fp32 absmax
    lb.absmax2 = rsrc(nullptr, 0);
  } else if constexpr (FMT == kFmtInt4) {
    lb.absmax_q = rsrc(d.absmax_q, static_cast<uint32_t>(nb * 2));  // fp16 group scales
    lb.absmax2 = rsrc(d.absmax2, static_cast<uint32_t>(nb * 2));    // fp16 zero points
  } else {
    lb.absmax_q = rsrc(d.absmax_q, static_cast<uint32_t>(nb));
    lb.absmax2 = rsrc(d.absmax2, static_cast<uint32_t>(ng * 2));
  }
  return lb;
}

template <int B>
__device__ __forceinline__ OutBufs out_bufs(const nf4_gemv_desc& d) {
  OutBufs ob;
  ob.y = rsrc(d.y, static_cast<uint32_t>(B * d.N * 2));
  ob.N = static_cast<int>(d.N);
  ob.offset = d.offset;
  return ob;
}

template <int B>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_buf(const nf4_gemv_desc& d, int K) {
  return rsrc(d.x, static_cast<uint32_t>(B * K * 2));
}

// Loads of one row group for one lane: the 16-byte packed chunk, absmax_q
// and absmax2 of rows [rl, rl + len) (rows past len read as zeros).
template <int R, int FMT>
struct RowGroup {
  u32x4 pk[R];
  // at the loaded width: widened where they are used, so that the widening
  // is not hoisted to the loop latch, where it would wait for the loads
  typename ScaleBits<FMT>::type q[R];
  uint16_t a2[R];  // double-quantized format only
};

// Per-lane parts of the buffer offsets (constant for the whole kernel): the
// lane's byte offset inside a packed row and its activation byte offset, both
// pushed out of range for lanes past K (their activations then read as zero,
// so whatever codes they see contribute nothing).
struct LaneOffsets {
  uint32_t pk;
  uint32_t x;
  uint32_t k0;
};

template <int R, int FMT, int LW = 4>
__device__ __forceinline__ void load_row_group(RowGroup<R, FMT>& rg, const LoadBufs& mb, int rl,
                                               int len, const LaneOffsets& lo, int K, int log2bs,
                                               int log2s2) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    // row part of the offsets: wave-uniform, so it goes in the scalar offset
    const uint32_t row = static_cast<uint32_t>(rl + rr);
    const uint32_t srow = rr < len ? row * static_cast<uint32_t>(K >> 1) : kFar;
    const uint32_t sfar = rr < len ? 0u : kFar;
    const uint32_t blk = (row * static_cast<uint32_t>(K) + lo.k0) >> log2bs;
    if constexpr (LW == 4) {
      rg.pk[rr] = __builtin_amdgcn_raw_buffer_load_b128(mb.packed, lo.pk, srow, kStreamLoad);
    } else {  // 16 columns per lane: dwords 0 and 1
      const uint2 v = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(mb.packed, lo.pk, srow, kStreamLoad));
      rg.pk[rr] = u32x4{v.x, v.y, 0u, 0u};
    }
    if constexpr (FMT == kFmtAbsmax32) {
      rg.q[rr] = __builtin_amdgcn_raw_buffer_load_b32(mb.absmax_q, blk * 4u, sfar, 0);
    } else if constexpr (FMT == kFmtInt4) {
      rg.q[rr] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax_q, blk * 2u, sfar, 0);
      rg.a2[rr] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, blk * 2u, sfar, 0);
    } else {
      rg.q[rr] = __builtin_amdgcn_raw_buffer_load_b8(mb.absmax_q, blk, sfar, 0);
      rg.a2[rr] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, (blk >> log2s2) * 2u, sfar, 0);
    }
  }
}

// The lane's 8 LW activations per batch row (raw bf16 pairs; dwords j < LW).
template <int B, int LW = 4>
__device__ __forceinline__ void load_x(u32x4 (&xr)[B][4], __amdgpu_buffer_rsrc_t xb,
                                       const LaneOffsets& lo, int K) {
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < LW; ++j)
      xr[b][j] = __builtin_amdgcn_raw_buffer_load_b128(xb, lo.x + 16u * j,
                                                        static_cast<uint32_t>(b * K * 2), 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// part[rr][b] += sum over the 8 weights of dword j of row rr's chunk (columns
// 8 j .. 8 j + 7 of the lane) of weight * x.  Each table entry holds the two
// NF4 values of one packed byte as bf16 pairs hi = bf16(v) and lo = bf16(v -
// hi) (hi + lo is within 2^-16 |v| of v); an activation dword is already the
// matching bf16 pair (even column low), so two v_dot2c_f32_bf16 per byte do
// the four products with fp32 accumulation and no conversion.
template <int B, int R, int FMT>
__device__ __forceinline__ void dot_columns(const RowGroup<R, FMT>& rg, const u32x4 (&xr)[B][4], int j,
                                            uint32_t copy_off, const uint2* s_pairs,
                                            float (&part)[R][B]) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const uint32_t d = rg.pk[rr][j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // address bits 15..8 = byte i of d, bits 7..0 = copy offset (selector
      // 0x0C = zero byte, 4 = byte 0 of the first operand, i = byte i of d)
      const uint32_t addr = __builtin_amdgcn_perm(copy_off, d, 0x0C0C0004u | (uint32_t(i) << 8));
      if constexpr (FMT == kFmtInt4) {
        // one exact bf16 code pair: q x summed here, z sum(x) applied per piece
        const uint32_t t =
            *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_pairs) + addr);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const uint32_t xw = xr[b][j][i];
          part[rr][b] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2, t), __builtin_bit_cast(bf16x2, xw), part[rr][b], false);
        }
      } else {
        const uint2 t =
            *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(s_pairs) + addr);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          // copy the element out first: __builtin_bit_cast applied directly to
          // a vector-element lvalue reads element 0 whatever the index
          const uint32_t xw = xr[b][j][i];
          const bf16x2 xp = __builtin_bit_cast(bf16x2, xw);
          part[rr][b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, t.x), xp,
                                                        part[rr][b], false);
          part[rr][b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, t.y), xp,
                                                        part[rr][b], false);
        }
      }
    }
  }
}

// The fp32 table: entry b = (NF4[b >> 4], NF4[b & 15]) as fp32 bits, even
// column first, copies placed as in build_pair_table.
__device__ __forceinline__ void build_f32_pair_table(uint2* s_pairs, int tid, int nthreads) {
  for (int w = tid; w < 512; w += nthreads) {
    const int b = w & 255, half = w >> 8;
    const uint2 entry = make_uint2(__builtin_bit_cast(uint32_t, nf4_value(b >> 4)),
                                   __builtin_bit_cast(uint32_t, nf4_value(b & 15)));
#pragma unroll
    for (int k = 0; k < 16; ++k) s_pairs[b * kPairCopies + ((b + 16 * half + k) & 31)] = entry;
  }
}

// part[rr][b] += the lane's 8 LW weights of row rr times their activations
// in fp32: one table read per packed byte gives both NF4 values exactly, and
// each product is one fp32 FMA (a wave64 v_fma_f32 issues in about 2/3 of
// the time of a v_dot2c_f32_bf16, and one replaces the hi and lo dot2 pair).
template <int B, int R, int LW, int FMT>
__device__ __forceinline__ void dot_columns_f32(const RowGroup<R, FMT>& rg,
                                                const float (&xf)[B][8 * LW], uint32_t copy_off,
                                                const uint2* s_pairs, float (&part)[R][B]) {
  const char* tab = reinterpret_cast<const char*>(s_pairs);
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const uint32_t d = rg.pk[rr][j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t addr = __builtin_amdgcn_perm(copy_off, d, 0x0C0C0004u | (uint32_t(i) << 8));
        const uint2 t = *reinterpret_cast<const uint2*>(tab + addr);
        const float w0 = __builtin_bit_cast(float, t.x), w1 = __builtin_bit_cast(float, t.y);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          part[rr][b] = __builtin_fmaf(w0, xf[b][8 * j + 2 * i], part[rr][b]);
          part[rr][b] = __builtin_fmaf(w1, xf[b][8 * j + 2 * i + 1], part[rr][b]);
        }
      }
    }
}

// A descriptor the streaming kernel can read: 16-byte aligned packed weights
// and activations, non-NULL arrays, a row count that matches the row offsets
// and N * K < 2^31.  Matrices that fail this are skipped (y is not written).
template <int FMT>
__device__ __forceinline__ bool desc_usable(const nf4_gemv_desc& d, int rows, int K) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(d.packed) | reinterpret_cast<uintptr_t>(d.x);
  // every offset the kernel forms must stay below 2^30 (see kFar)
  const bool small = d.N >= 0 && static_cast<uint64_t>(d.N) * static_cast<uint64_t>(K) <
                                     (uint64_t(1) << 31);
  // the scale arrays: fp32 absmax 4-byte, fp16 scales and zero points 2-byte
  // aligned (the absmax_q bytes and absmax2 halves of the double format too)
  const uintptr_t sa = reinterpret_cast<uintptr_t>(d.absmax_q);
  const uintptr_t za = reinterpret_cast<uintptr_t>(d.absmax2);
  const bool scales_ok = FMT == kFmtAbsmax32 ? (sa & 3) == 0
                         : FMT == kFmtInt4   ? ((sa | za) & 1) == 0
                                             : (za & 1) == 0;
  return (a & 15) == 0 && d.N == rows && small && d.packed && d.absmax_q &&
         (FMT == kFmtAbsmax32 || d.absmax2) && d.x && d.y && scales_ok;
}

// Field-wise copy of descriptor m (or of the by-value descriptor when the
// list is absent).  m is wave-uniform, so these become scalar loads; copying
// the struct as a whole would go through scratch memory.
__device__ __forceinline__ nf4_gemv_desc fetch_desc(const nf4_gemv_desc* __restrict__ descs,
                                                    const nf4_gemv_desc& single, int m) {
  nf4_gemv_desc d;
  if (descs == nullptr || m < 0) {
    d.packed = single.packed;
    d.absmax_q = single.absmax_q;
    d.absmax2 = single.absmax2;
    d.x = single.x;
    d.y = single.y;
    d.N = single.N;
    d.offset = single.offset;
  } else {
    const nf4_gemv_desc* p = descs + m;
    d.packed = p->packed;
    d.absmax_q = p->absmax_q;
    d.absmax2 = p->absmax2;
    d.x = p->x;
    d.y = p->y;
    d.N = p->N;
    d.offset = p->offset;
  }
  d.row_begin = 0;
  d.reserved = 0;
  return d;
}

// An LDS read at a wave-uniform index: the value is uniform too.  Saying so
// keeps the cursor in scalar registers; otherwise the row offsets derived from
// it are assumed divergent and every buffer load whose scalar offset uses them
// is wrapped in a loop over distinct values.
__device__ __forceinline__ int uniform_lds(const int* p, int i) {
  return __builtin_amdgcn_readfirstlane(p[i]);
}

// Row offsets of the matrices (row_begin, with total_rows after the last):
// read from LDS for a descriptor list; for a single matrix they are just 0 and
// N, and no LDS read (a round trip on the kernel's critical path) is made.
struct RowBegins {
  const int* lds;  // nullptr: a single matrix
  int total;
  __device__ __forceinline__ int operator()(int m) const {
    return lds != nullptr ? uniform_lds(lds, m) : (m <= 0 ? 0 : total);
  }
};

// Descriptor m for the kernel: a matrix it cannot use (see desc_usable) is
// replaced by an empty one, whose loads read zeros and whose stores are
// dropped.
template <int FMT>
__device__ __forceinline__ nf4_gemv_desc open_desc(const nf4_gemv_desc* __restrict__ descs,
                                                   const nf4_gemv_desc& single, int m, int len,
                                                   const RowBegins& rbeg, int K) {
  nf4_gemv_desc d = fetch_desc(descs, single, m);
  if (len <= 0 || m < 0 ||
      !desc_usable<FMT>(d, rbeg(m + 1) - rbeg(m), K)) {
    d.packed = nullptr;
    d.absmax_q = nullptr;
    d.absmax2 = nullptr;
    d.x = nullptr;
    d.y = nullptr;
    d.N = 0;
    d.offset = 0.0f;
  }
  return d;
}

// Part i of `total` rows split as evenly as possible into `parts` contiguous
// ranges (the first total % parts ranges hold one row more): [*lo, *hi).  All
// 32-bit, so that wave-uniform operands stay a few scalar instructions (a
// 64-bit division is a long emulated sequence on the scalar unit).
__device__ __forceinline__ void split_rows(uint32_t total, uint32_t parts, uint32_t i, int* lo,
                                           int* hi) {
  const uint32_t q = total / parts, rem = total - q * parts;
  const uint32_t b = i * q + (i < rem ? i : rem);
  *lo = static_cast<int>(b);
  *hi = static_cast<int>(b + q + (i < rem ? 1u : 0u));
}

// Where a team is in the concatenated row space: matrix m, global row r.
struct RowCursor {
  int m;      // current matrix
  int r;      // next global row
  int beg;    // first global row of matrix m
  int end;    // one past its last row
};

// The next group of at most R rows from cursor c, not crossing a matrix end or
// the team's range end; advances c.  Returns the group's length (0 when the
// range is exhausted).  The row offsets in LDS are read only when the cursor
// moves to another matrix.
template <int R>
__device__ __forceinline__ int next_group(RowCursor& c, int r_end, const RowBegins& rbeg, int count,
                                          int* m_out, int* rl_out) {
  if (c.r >= c.end && c.r < r_end) {  // skip finished / empty matrices
    while (c.m < count && rbeg(c.m + 1) <= c.r) ++c.m;
    c.beg = c.m < count ? rbeg(c.m) : c.r;
    c.end = c.m < count ? rbeg(c.m + 1) : c.r;
  }
  if (c.r >= r_end || c.r >= c.end) {
    *m_out = -1;
    *rl_out = 0;
    return 0;
  }
  const int len = min(R, min(r_end, c.end) - c.r);
  *m_out = c.m;
  *rl_out = c.r - c.beg;
  c.r += len;
  return len;
}

// ---------------------------------------------------------------------------
// The streaming GEMV kernel: one launch over a list of matrices that share K,
// the block sizes, code2 and the batch (a single nf4_gemv is a list of one).
// The concatenated rows of all matrices are split evenly into contiguous
// ranges, one per team; a team walks its range in groups of up to R rows
// (never crossing a matrix), issuing the loads of the next group before it
// computes the current one.  All loads and the y stores are branch-free
// buffer operations.
// ---------------------------------------------------------------------------
// SINGLE: one matrix given by value (descs NULL, count 1), known at compile
// time: no descriptor walk, no matrix or activation switches, so the loop
// keeps far less scalar state.
// LW: packed dwords per lane (8 LW columns, slabs of 512 LW columns).
// XF (with LW = 2, one matrix at batch 3-8): the table holds each byte's two
// NF4 values as exact fp32, the activations are widened to fp32 once, and
// every product is one fp32 FMA instead of the hi and lo dot2 pair.
template <int B, int R, int NW, int WPE, int FMT = kFmtDouble, bool SINGLE = false, int LW = 4,
          bool XF = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemv_stream_kernel(
    const nf4_gemv_desc* __restrict__ descs, nf4_gemv_desc single, int count, int total_rows,
    int K, int log2bs, int log2s2, const uint16_t* __restrict__ code2) {
  constexpr int nw = NW;  // waves per team: one per slab of 512 LW columns of K
  // (XF widens the activations once: a launch over several matrices would
  // have to widen them again at every switch)
  static_assert(!XF || (SINGLE && LW == 2 && FMT == kFmtDouble),
                "fp32 products: one matrix, NF4 codes, 16 columns per lane");
  if constexpr (SINGLE) {
    descs = nullptr;
    count = 1;
  }
  __shared__ uint2 s_pairs[256 * kPairCopies];  // 64 KiB decode table
  __shared__ float s_code2[256];
  __shared__ float s_red[2][8][R * B];
  __shared__ int s_rowbeg[kMaxDescs + 1];
  __shared__ int s_iters;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; saying so keeps all per-team bookkeeping
  // in scalar registers and scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // code2 is fetched first and written to LDS only after the row loads are
  // issued: its wait then overlaps theirs (the launch uses 512 threads)
  // (a bounds-checked load for all lanes: lanes past the table read 0)
  const uint16_t code2_bits = __builtin_amdgcn_raw_buffer_load_b16(
      rsrc(FMT == kFmtDouble ? code2 : nullptr, 512), static_cast<uint32_t>(tid) * 2u, 0u, 0);
  constexpr int teams = 8 / NW;         // the workgroup has 8 waves
  const int team = wave / nw;           // == teams for helper waves
  const int slab = wave - team * nw;
  const bool in_team = team < teams;
  const int k0 = slab * (512 * LW) + lane * (8 * LW);
  const bool active = in_team && k0 < K;

  // descriptor row offsets, code2 and the NF4 table into LDS
  if (descs == nullptr) {
    if (tid == 0) s_rowbeg[0] = 0;
  } else {
    for (int i = tid; i < count; i += blockDim.x) s_rowbeg[i] = static_cast<int>(descs[i].row_begin);
  }
  if (tid == 0) {
    s_rowbeg[count] = total_rows;
    s_iters = 0;
  }
  __syncthreads();
  const RowBegins rbeg{descs != nullptr ? s_rowbeg : nullptr, total_rows};

  // the team's row range
  int r_begin = 0, r_end = 0;
  if (in_team)
    split_rows(static_cast<uint32_t>(total_rows), gridDim.x * static_cast<uint32_t>(teams),
               blockIdx.x * static_cast<uint32_t>(teams) + static_cast<uint32_t>(team), &r_begin,
               &r_end);
  RowCursor cur_c;
  {
    int lo = 0, hi = count - 1;  // last matrix whose first row is <= r_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rbeg(mid) <= r_begin) lo = mid; else hi = mid - 1;
    }
    cur_c.m = lo;
    cur_c.r = r_begin;
    cur_c.beg = rbeg(lo);
    cur_c.end = rbeg(lo + 1);
  }
  // number of groups of this team (per matrix it overlaps), then the
  // workgroup maximum: every wave runs that many iterations
  {
    int ng = 0;
    if constexpr (SINGLE) {
      ng = (r_end - r_begin + R - 1) / R;
    } else {
      for (int mm = cur_c.m; mm < count && rbeg(mm) < r_end; ++mm) {
        const int lo = max(r_begin, rbeg(mm));
        const int hi = min(r_end, rbeg(mm + 1));
        if (hi > lo) ng += (hi - lo + R - 1) / R;
      }
    }
    if (lane == 0 && slab == 0 && in_team) atomicMax(&s_iters, ng);
  }
  // the next group of the team's range: a single matrix needs no cursor walk
  auto advance = [&](int* m_out, int* rl_out) {
    if constexpr (SINGLE) {
      const int len = cur_c.r < r_end ? min(R, r_end - cur_c.r) : 0;
      *m_out = len > 0 ? 0 : -1;
      *rl_out = cur_c.r;
      cur_c.r += len;
      return len;
    } else {
      return next_group<R>(cur_c, r_end, rbeg, count, m_out, rl_out);
    }
  };

  // the first two groups (prefetch depth 2: the loads of group i + 2 are
  // issued before group i is computed).  Scalar state: the load-side buffers
  // of the newest group's matrix (mL), and the output side of the two groups
  // in compute order; descriptors are re-read only when the matrix changes.
  int m0, rl0, m1, rl1;
  int len0 = advance(&m0, &rl0);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  // a single matrix: the whole team range's descriptor (valid for any length)
  const nf4_gemv_desc d0 = SINGLE ? open_desc<FMT>(nullptr, single, 0, total_rows, rbeg, K)
                                  : open_desc<FMT>(descs, single, m0, len0, rbeg, K);
  int len1 = advance(&m1, &rl1);
  m1 = __builtin_amdgcn_readfirstlane(m1);
  LoadBufs lb0 = load_bufs<FMT>(d0, K, log2bs, log2s2);
  OutBufs ob0 = out_bufs<B>(d0);
  LaneOffsets lo;
  lo.pk = active ? static_cast<uint32_t>(k0 >> 1) : kFar;
  lo.x = active ? static_cast<uint32_t>(k0 * 2) : kFar;
  lo.k0 = static_cast<uint32_t>(k0);
  RowGroup<R, FMT> g0, g1;
  load_row_group<R, FMT, LW>(g0, lb0, rl0, len0, lo, K, log2bs, log2s2);
  u32x4 xr[B][4];
  load_x<B, LW>(xr, x_buf<B>(d0, K), lo, K);
  float xs[B];  // INT4: the lane's activation sums (computed before the loop)
  int mL = m0;            // matrix of lbL
  LoadBufs lbL = lb0;
  OutBufs ob1 = ob0;
  if (!SINGLE && len1 > 0 && m1 != m0) {
    const nf4_gemv_desc d1 = open_desc<FMT>(descs, single, m1, len1, rbeg, K);
    lbL = load_bufs<FMT>(d1, K, log2bs, log2s2);
    ob1 = out_bufs<B>(d1);
    mL = m1;
  }
  load_row_group<R, FMT, LW>(g1, lbL, rl1, len1, lo, K, log2bs, log2s2);

  // the 256 x 32 pair table: (bf16 hi pair, bf16 lo pair) of each byte
  if (FMT == kFmtDouble && tid < 256) s_code2[tid] = f16_to_f32(code2_bits);
  uint32_t copy_off;
  if constexpr (XF) {
    build_f32_pair_table(s_pairs, tid, blockDim.x);
    copy_off = static_cast<uint32_t>(lane % kPairCopies) * 8u;
  } else {
    copy_off = build_decode_table<FMT>(s_pairs, tid, blockDim.x, lane);
  }
  // XF: the lane's activations widened to fp32 once (even column: low half)
  float xf[XF ? B : 1][XF ? 8 * LW : 1];
  if constexpr (XF) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
#pragma unroll
      for (int j = 0; j < LW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = xr[bb][j][i];
          xf[bb][8 * j + 2 * i] = __builtin_bit_cast(float, w << 16);
          xf[bb][8 * j + 2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
        }
  }
  auto sum_x = [&]() {
    if constexpr (FMT == kFmtInt4) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        uint32_t w[4 * LW];
#pragma unroll
        for (int j = 0; j < LW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) w[4 * j + i] = xr[b][j][i];
        xs[b] = pair_sum(w);
      }
    }
  };
  sum_x();
  __syncthreads();
  const int iters = __builtin_amdgcn_readfirstlane(s_iters);

  // One iteration: issue the loads of the group after next into `fut` (the
  // buffer the previous iteration computed from), then compute `cur`.  The
  // loop is unrolled by three so that the three buffers change roles without
  // register copies: a copy out of a buffer whose loads are in flight would
  // wait for them, and the prefetch would be lost.
  int buf = 0;
  auto step = [&](RowGroup<R, FMT>& cur, RowGroup<R, FMT>& fut) {
    int m2, rl2;
    const int len2 = advance(&m2, &rl2);
    m2 = __builtin_amdgcn_readfirstlane(m2);
    OutBufs ob2 = ob1;
    if (!SINGLE && len2 > 0 && m2 != mL) {
      const nf4_gemv_desc d2 = open_desc<FMT>(descs, single, m2, len2, rbeg, K);
      lbL = load_bufs<FMT>(d2, K, log2bs, log2s2);
      ob2 = out_bufs<B>(d2);
      mL = m2;
    }
    load_row_group<R, FMT, LW>(fut, lbL, rl2, len2, lo, K, log2bs, log2s2);
    // issue these loads here: sunk below the first wait for the current group
    // they would turn that wait into a wait for the group after it as well
    __builtin_amdgcn_sched_barrier(0);

    float c2[R];
    if constexpr (FMT == kFmtDouble) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) c2[rr] = s_code2[cur.q[rr]];
    }
    float part[R][B];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int b = 0; b < B; ++b) part[rr][b] = 0.0f;
    if constexpr (XF) {
      dot_columns_f32<B, R, LW, FMT>(cur, xf, copy_off, s_pairs, part);
    } else {
#pragma unroll
      for (int j = 0; j < LW; ++j) dot_columns<B, R, FMT>(cur, xr, j, copy_off, s_pairs, part);
    }
    float val[R * B];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      if constexpr (FMT == kFmtInt4) {
        const float sc = f16_to_f32(cur.q[rr]);
        const float z = f16_to_f32(cur.a2[rr]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float zt = z * xs[b];
          val[rr * B + b] = sc * (part[rr][b] - zt);
        }
      } else {
        float a;
        if constexpr (FMT == kFmtAbsmax32) {
          a = __builtin_bit_cast(float, cur.q[rr]);
        } else {
          const float prod = c2[rr] * f16_to_f32(cur.a2[rr]);
          a = prod + ob0.offset;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) val[rr * B + b] = a * part[rr][b];
      }
    }
    if constexpr (R * B == 2) {
      const float tot = wave_sum_pair(val[0], val[1]);
      if ((lane & 31) == 0) s_red[buf][wave][lane >> 5] = tot;
    } else {
      // four values at a time; 16-lane row r holds value 4 q + 2 (r & 1) + (r >> 1)
      const int row16 = lane >> 4;
      const int slot = ((row16 & 1) << 1) | (row16 >> 1);
#pragma unroll
      for (int q = 0; q < (R * B + 3) / 4; ++q) {
        const float tot = wave_sum_quad(val[4 * q], 4 * q + 1 < R * B ? val[4 * q + 1] : 0.0f,
                                        4 * q + 2 < R * B ? val[4 * q + 2] : 0.0f,
                                        4 * q + 3 < R * B ? val[4 * q + 3] : 0.0f);
        if ((lane & 15) == 0 && 4 * q + slot < R * B) s_red[buf][wave][4 * q + slot] = tot;
      }
    }
    __syncthreads();
    {
      const int idx = lane < R * B ? lane : 0;
      const int rr = idx / B, b = idx % B;
      float acc = s_red[buf][wave][idx];
#pragma unroll
      for (int w = 1; w < NW; ++w) acc += s_red[buf][min(wave + w, 7)][idx];
      const bool store = in_team && slab == 0 && lane < R * B && rr < len0;
      const uint32_t off = static_cast<uint32_t>((b * ob0.N + rl0 + rr) * 2);
      __builtin_amdgcn_raw_buffer_store_b16(to_half_bits<NF4_BF16>(acc), ob0.y,
                                            store ? off : kOutOfRange, 0, 0);
    }
    buf ^= 1;
    // the next group starts a new matrix: fetch its activations now that the
    // current ones are no longer needed
    if (!SINGLE && len1 > 0 && m1 != m0) {
      load_x<B, LW>(xr, x_buf<B>(open_desc<FMT>(descs, single, m1, len1, rbeg, K), K), lo, K);
      // drain here (rare: once per matrix change) so that the loads of this
      // branch are not assumed outstanding on the common path, where they
      // would make every wait for the current group also wait for the next
      __builtin_amdgcn_s_waitcnt(0);
      sum_x();
    }
    ob0 = ob1;
    ob1 = ob2;
    m0 = len1 > 0 ? m1 : m0;
    m1 = len2 > 0 ? m2 : m1;
    rl0 = rl1;
    rl1 = rl2;
    len0 = len1;
    len1 = len2;
  };
  // Whole rounds of three steps in the loop, the remaining steps after it: an
  // exit from the middle of a round would give the compiler a path from that
  // step back to the loop header, and loads still counted on it would make
  // the first step wait for the loads it has just issued.
  RowGroup<R, FMT> g2;
  const int rounds = iters / 3;
  for (int it = 0; it < rounds; ++it) {
    step(g0, g2);
    step(g1, g0);
    step(g2, g1);
  }
  const int rest = iters - 3 * rounds;
  if (rest > 0) step(g0, g2);
  if (rest > 1) step(g1, g0);
}

// ---------------------------------------------------------------------------
// The wave-per-row streaming GEMV (K a multiple of 64, blocksize >= 64).
//
// Every wave works alone.  Pass p < P (P = ceil(K / 4096)) covers the columns
// [4096 p, +4096) of a row, 2 KiB of packed bytes, read by two 16-byte loads
// per lane: load h (h = 0, 1) of lane l takes the 32 columns
// [4096 p + 2048 h + 32 l, +32), so each load instruction of the wave reads
// one contiguous KiB (a lane-strided pair of loads that each cover half of
// every line reads about a fifth slower on this part).  A 32-column piece lies
// inside one first-level block, so lanes 2j and 2j+1 hold the two halves of
// block j of the pass (first load) and of block 32 + j (second load).  Each
// lane sums its 32 products per load; one DPP swap inside the lane pair adds
// the partner's half, after which lane 2j holds the sum of block j and lane
// 2j+1 that of block 32 + j.  So each lane still loads one absmax_q / absmax2
// pair per row and pass -- that of the block it finishes -- and applies one
// absmax_real to the block's 64-product sum.  A wave reduces its own rows (no
// cross-wave sums, no barriers), so the waves of a workgroup share only the
// decode table and code2.  The concatenated rows of all matrices are split
// evenly into contiguous ranges, one per wave; a wave walks its range in
// groups of up to R rows with the loads of the group after next issued before
// the current group is computed (three register buffers, loop unrolled by
// three).
// ---------------------------------------------------------------------------
constexpr int kWaveCols = 4096;  // columns per pass of a wave (2 loads x 64 lanes x 32)

template <int R, int P, int FMT>
struct WaveGroup {
  u32x4 pk[R][P][2];
  typename ScaleBits<FMT>::type q[R][P];
  uint16_t a2[R][P];  // double-quantized format only
};

// Per-lane offsets of load h of pass p: packed byte offset inside a row and
// activation byte offset (pushed out of range when the load's columns are past
// K), and the first column of the block the lane finishes in pass p.
template <int P>
struct WaveLane {
  uint32_t pk[P][2];
  uint32_t x[P][2];
  uint32_t c0[P];
  // regular shapes (see load_wave_group): the lane's block and group inside
  // its row, and the byte offsets of its scale entries relative to the row's
  uint32_t sq[P], sa2[P];
};

// REG (regular shapes: K a multiple of the block size, and the blocks of a
// row and the s2 blocks of a group dividing one into the other): a row's first
// block and first group are then the same for all lanes, so the row part of
// every scale offset is wave-uniform and goes into the scalar offset, and the
// lane's part is a constant (wl.sq, wl.sa2).  Otherwise the lane forms its
// block index per row.
template <int R, int P, int FMT, bool REG = false>
__device__ __forceinline__ void load_wave_group(WaveGroup<R, P, FMT>& g, const LoadBufs& mb, int rl,
                                                int len, const WaveLane<P>& wl, int K, int log2bs,
                                                int log2s2) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const uint32_t row = static_cast<uint32_t>(rl + rr);
    const uint32_t srow = rr < len ? row * static_cast<uint32_t>(K >> 1) : kFar;
    const uint32_t sfar = rr < len ? 0u : kFar;
    if constexpr (REG) {
      const uint32_t rb = row * static_cast<uint32_t>(K >> log2bs);  // the row's first block
      const uint32_t sq = rr < len ? rb * (FMT == kFmtAbsmax32 ? 4u : FMT == kFmtInt4 ? 2u : 1u)
                                   : kFar;
      const uint32_t sa = rr < len ? (FMT == kFmtInt4 ? rb * 2u : (rb >> log2s2) * 2u) : kFar;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        g.pk[rr][p][0] = __builtin_amdgcn_raw_buffer_load_b128(mb.packed, wl.pk[p][0], srow,
                                                                kStreamLoad);
        g.pk[rr][p][1] = __builtin_amdgcn_raw_buffer_load_b128(mb.packed, wl.pk[p][1], srow,
                                                                kStreamLoad);
        if constexpr (FMT == kFmtAbsmax32) {
          g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b32(mb.absmax_q, wl.sq[p], sq, 0);
        } else if constexpr (FMT == kFmtInt4) {
          g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax_q, wl.sq[p], sq, 0);
          g.a2[rr][p] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, wl.sa2[p], sa, 0);
        } else {
          g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b8(mb.absmax_q, wl.sq[p], sq, 0);
          g.a2[rr][p] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, wl.sa2[p], sa, 0);
        }
      }
      continue;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t blk = (row * static_cast<uint32_t>(K) + wl.c0[p]) >> log2bs;
      g.pk[rr][p][0] = __builtin_amdgcn_raw_buffer_load_b128(mb.packed, wl.pk[p][0], srow,
                                                              kStreamLoad);
      g.pk[rr][p][1] = __builtin_amdgcn_raw_buffer_load_b128(mb.packed, wl.pk[p][1], srow,
                                                              kStreamLoad);
      if constexpr (FMT == kFmtAbsmax32) {
        g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b32(mb.absmax_q, blk * 4u, sfar, 0);
      } else if constexpr (FMT == kFmtInt4) {
        g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax_q, blk * 2u, sfar, 0);
        g.a2[rr][p] = __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, blk * 2u, sfar, 0);
      } else {
        g.q[rr][p] = __builtin_amdgcn_raw_buffer_load_b8(mb.absmax_q, blk, sfar, 0);
        g.a2[rr][p] =
            __builtin_amdgcn_raw_buffer_load_b16(mb.absmax2, (blk >> log2s2) * 2u, sfar, 0);
      }
    }
  }
}

// The lane's 64 activations per pass and batch row (raw bf16 pairs): xr[.][p]
// [0..3] are the 32 columns of load 0, [4..7] those of load 1.
template <int B, int P>
__device__ __forceinline__ void load_wave_x(u32x4 (&xr)[B][P][8], __amdgpu_buffer_rsrc_t xb,
                                            const WaveLane<P>& wl, int K) {
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        xr[b][p][j] = __builtin_amdgcn_raw_buffer_load_b128(xb, wl.x[p][j >> 2] + 16u * (j & 3),
                                                             static_cast<uint32_t>(b * K * 2), 0);
}

// Sum over a lane pair (2j, 2j+1) with DPP quad_perm [1,0,3,2]; both lanes get
// the same bits (the add is commutative).
__device__ __forceinline__ float pair_lane_sum(float v) { return dpp_add<0xB1, 0xF>(v); }

// val[rr * B + b] = the lane's share of row rr of weight * x.  The lane's
// R P 8 packed dwords are walked in order with the four table reads of the
// next dword issued before the eight v_dot2c_f32_bf16 of the current one
// (same decode table as the team kernel); the scheduling barriers keep the
// compiler from hoisting more reads, whose results would not fit in
// registers.  Each load's 32 products are summed on their own; at the end of
// a (row, pass) the two half sums of each block are completed across the lane
// pair, and the lane scales the block it owns (odd lanes: the second load's)
// by its absmax_real.
//
// XL: the activations come from the workgroup's LDS copy s_x (lane-major:
// the 8 columns of dword hj of pass p for batch row b and lane l at
// s_x[((b P + p) 8 + hj) 64 + l]), read with the table entries one dword
// ahead, instead of from the registers xr.
template <int B, int R, int P, int FMT, bool XL = false>
__device__ __forceinline__ void wave_rows(const WaveGroup<R, P, FMT>& g, const u32x4 (&xr)[B][P][8],
                                          uint32_t copy_off, const uint2* s_pairs,
                                          const float* s_code2, float offset, bool odd,
                                          const bool (&own_in)[P], const float (&xs)[B][P],
                                          float (&val)[R * B], const u32x4* s_x = nullptr,
                                          int lane = 0) {
  constexpr int U = R * P * 8;
  const char* tab = reinterpret_cast<const char*>(s_pairs);
  uint2 t[2][4];
  u32x4 xv[2][B];
  auto fetch = [&](int u, uint2 (&tt)[4], u32x4 (&xx)[B]) {
    const int rr = u / (P * 8), p = (u / 8) % P, hj = u % 8;
    const uint32_t d = g.pk[rr][p][hj >> 2][hj & 3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t addr = __builtin_amdgcn_perm(copy_off, d, 0x0C0C0004u | (uint32_t(i) << 8));
      if constexpr (FMT == kFmtInt4)
        tt[i].x = *reinterpret_cast<const uint32_t*>(tab + addr);  // one exact code pair
      else
        tt[i] = *reinterpret_cast<const uint2*>(tab + addr);
    }
    if constexpr (XL) {
#pragma unroll
      for (int b = 0; b < B; ++b) xx[b] = s_x[((b * P + p) * 8 + hj) * 64 + lane];
    }
  };
  float part[B], half0[B];
  fetch(0, t[0], xv[0]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u + 1 < U) fetch(u + 1, t[(u + 1) & 1], xv[(u + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    const int rr = u / (P * 8), p = (u / 8) % P, hj = u % 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 ti = t[u & 1][i];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        // copied out first: a bit_cast of a vector-element lvalue reads
        // element 0 whatever the index
        const uint32_t xw = XL ? xv[u & 1][b][i] : xr[b][p][hj][i];
        const bf16x2 xp = __builtin_bit_cast(bf16x2, xw);
        // the first product of each half starts from an immediate zero (no
        // separate reset of the accumulator)
        const float acc = (hj & 3) == 0 && i == 0 ? 0.0f : part[b];
        part[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ti.x), xp, acc,
                                                  false);
        if constexpr (FMT != kFmtInt4)
          part[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ti.y), xp,
                                                    part[b], false);
      }
    }
    if (hj == 3) {
#pragma unroll
      for (int b = 0; b < B; ++b) half0[b] = part[b];
    }
    if (hj == 7) {
      // the 64-product sum of the lane's block: its own half plus the
      // partner's half of the same load
      float blk[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float s0 = pair_lane_sum(half0[b]);
        const float s1 = pair_lane_sum(part[b]);
        blk[b] = odd ? s1 : s0;
      }
      if constexpr (FMT == kFmtInt4) {
        // s (sum q x - z sum x) over the 64 columns of one group
        const float sc = f16_to_f32(g.q[rr][p]);
        const float z = f16_to_f32(g.a2[rr][p]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float zt = z * xs[b][p];
          const float c = own_in[p] ? sc * (blk[b] - zt) : 0.0f;
          val[rr * B + b] = p == 0 ? c : val[rr * B + b] + c;  // the first pass assigns
        }
      } else {
        float a;
        if constexpr (FMT == kFmtAbsmax32) {
          a = __builtin_bit_cast(float, g.q[rr][p]);
        } else {
          const float prod = s_code2[g.q[rr][p]] * f16_to_f32(g.a2[rr][p]);
          a = prod + offset;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float c = own_in[p] ? a * blk[b] : 0.0f;
          val[rr * B + b] = p == 0 ? c : val[rr * B + b] + c;  // the first pass assigns
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Dynamic row distribution.  The rows are split into `nreg` equal regions
// (workgroup b serves region b % nreg: with the usual round-robin placement
// of workgroups on the XCDs, one region per XCD, so the claims of a region
// stay on one L2).  Inside a region the rows go out in chunks of C: wave w of
// the region starts with chunk w, and the chunks after the first W go to
// whichever wave claims them from the region's counter.  Each wave claims one
// chunk ahead (the claim's result is read only when the current chunk is
// done).  Waves on one SIMD are not issued fairly (the older wave wins), so a
// static split leaves the younger waves with the tail; the rotating wave
// priority (rotate_priority) evens out most of it and the claimed chunks the
// rest.
struct SchedRegion {
  unsigned* claims;  // claims made on this region (kept by the workspace)
  unsigned* done;    // waves of this region that have finished
  int lo, hi;        // rows of the region
  int dyn_lo;        // first row handed out in chunks (after the static shares)
  int W;             // waves serving the region
};
constexpr int kSchedStride = 64;  // uint32 per region (256 bytes): counters on separate lines
constexpr int kSchedRegions = 8;

// The claim of the next chunk, issued by lane 0 only; the other lanes keep
// their value, so nothing else writes the register while the atomic is in
// flight.
__device__ __forceinline__ void claim_chunk(uint32_t& claim, unsigned* claims, int lane) {
  if (lane == 0) claim = atomicAdd(claims, 1u);
}

// next_group over a chunked range: when the current chunk [c.r, r_end) is
// used up, the pre-claimed chunk W + claim is taken (and the next one
// claimed), or the wave's range ends at the region's end.
template <int R>
__device__ __forceinline__ int next_group_dyn(RowCursor& c, int& r_end, uint32_t& claim,
                                              const SchedRegion& sr, int C, int log2C,
                                              const RowBegins& rbeg,
                                              int count, int lane, int* m_out, int* rl_out) {
  if (c.r >= r_end && r_end < sr.hi) {
    // read at the use, not hoisted next to the atomic: an early read would
    // wait for every load issued before the atomic
    uint32_t cl;
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(cl) : "v"(claim));
    const uint32_t ch = cl;
    const uint32_t nch =
        (static_cast<uint32_t>(sr.hi - sr.dyn_lo) + static_cast<uint32_t>(C) - 1u) >> log2C;
    if (ch >= nch) {
      c.r = r_end = sr.hi;
    } else {
      c.r = sr.dyn_lo + static_cast<int>(ch << log2C);
      r_end = min(c.r + C, sr.hi);
      if (r_end < sr.hi) claim_chunk(claim, sr.claims, lane);
    }
  }
  return next_group<R>(c, r_end, rbeg, count, m_out, rl_out);
}

// Rotating wave priority.  A SIMD issues its ready waves oldest first, so
// with equal priorities the younger waves of a SIMD fall behind and finish
// last.  Each round of three row groups a wave moves its priority one level
// (0-3) along a cycle that starts at its wave slot on the SIMD, so the waves
// of a SIMD take turns at the top and progress evenly.  (A wave's issue
// priority only: the queue and its streams keep the default priority.)
constexpr int kHwRegWaveSlot = 4 | (0 << 6) | (3 << 11);  // HW_ID bits 3:0, the wave's slot
__device__ __forceinline__ void rotate_priority(int round, int slot) {
  const int lvl = __builtin_amdgcn_readfirstlane((round + slot) & 3);
  if (lvl == 0)
    __builtin_amdgcn_s_setprio(0);
  else if (lvl == 1)
    __builtin_amdgcn_s_setprio(1);
  else if (lvl == 2)
    __builtin_amdgcn_s_setprio(2);
  else
    __builtin_amdgcn_s_setprio(3);
}

template <int B, int R, int P, int WPE, bool DYN, int FMT = kFmtDouble, bool REG = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemv_wave_kernel(
    const nf4_gemv_desc* __restrict__ descs, nf4_gemv_desc single, int count, int total_rows,
    int K, int log2bs, int log2s2, const uint16_t* __restrict__ code2, unsigned* sched, int C,
    int S) {
  static_assert(R * B <= 4, "one pair or quad reduction per group");
  const int log2C = C > 0 ? __builtin_ctz(static_cast<unsigned>(C)) : 0;  // C is a power of two
  __shared__ uint2 s_pairs[256 * kPairCopies];  // 64 KiB decode table
  __shared__ float s_code2[256];
  __shared__ int s_rowbeg[kMaxDescs + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // code2 is fetched first and written to LDS only after the row loads are
  // issued: its wait then overlaps theirs (the launch uses 512 threads)
  // (a bounds-checked load for all lanes: lanes past the table read 0)
  const uint16_t code2_bits = __builtin_amdgcn_raw_buffer_load_b16(
      rsrc(FMT == kFmtDouble ? code2 : nullptr, 512), static_cast<uint32_t>(tid) * 2u, 0u, 0);

  if (descs == nullptr) {
    if (tid == 0) s_rowbeg[0] = 0;
  } else {
    for (int i = tid; i < count; i += blockDim.x) s_rowbeg[i] = static_cast<int>(descs[i].row_begin);
  }
  if (tid == 0) s_rowbeg[count] = total_rows;
  __syncthreads();
  const RowBegins rbeg{descs != nullptr ? s_rowbeg : nullptr, total_rows};

  // the wave's rows: a fixed share, or its first chunk (DYN)
  const int waves = blockDim.x >> 6;
  int r_begin, r_end;
  SchedRegion sr{};
  uint32_t claim = 0;
  if constexpr (DYN) {
    const int nreg = min(kSchedRegions, static_cast<int>(gridDim.x));
    const int region = static_cast<int>(blockIdx.x) % nreg;
    sr.claims = sched + region * kSchedStride;
    sr.done = sr.claims + 1;
    split_rows(static_cast<uint32_t>(total_rows), static_cast<uint32_t>(nreg),
               static_cast<uint32_t>(region), &sr.lo, &sr.hi);
    sr.W = waves * ((static_cast<int>(gridDim.x) - 1 - region) / nreg + 1);
    const int wr = (static_cast<int>(blockIdx.x) / nreg) * waves + wave;  // index in the region
    const uint32_t rows = static_cast<uint32_t>(sr.hi - sr.lo);
    // a contiguous static share of S rows per wave first (wr < 2^13, S < 2^18),
    // then chunks of C from the rest of the region
    const uint32_t first = static_cast<uint32_t>(wr) * static_cast<uint32_t>(S);
    const uint32_t shares = static_cast<uint32_t>(sr.W) * static_cast<uint32_t>(S);
    sr.dyn_lo = sr.lo + static_cast<int>(shares < rows ? shares : rows);
    r_begin = sr.lo + static_cast<int>(first < rows ? first : rows);
    r_end = sr.lo + static_cast<int>(first + S < rows ? first + S : rows);
    if (r_end < sr.hi) claim_chunk(claim, sr.claims, lane);
  } else {
    split_rows(static_cast<uint32_t>(total_rows), gridDim.x * static_cast<uint32_t>(waves),
               blockIdx.x * static_cast<uint32_t>(waves) + static_cast<uint32_t>(wave), &r_begin,
               &r_end);
  }
  RowCursor cur_c;
  {
    int lo = 0, hi = count - 1;  // last matrix whose first row is <= r_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rbeg(mid) <= r_begin) lo = mid; else hi = mid - 1;
    }
    cur_c.m = lo;
    cur_c.r = r_begin;
    cur_c.beg = rbeg(lo);
    cur_c.end = rbeg(lo + 1);
  }
  // groups of this wave (static split only)
  int iters = 0;
  for (int mm = cur_c.m; !DYN && mm < count && rbeg(mm) < r_end; ++mm) {
    const int lo = max(r_begin, rbeg(mm));
    const int hi = min(r_end, rbeg(mm + 1));
    if (hi > lo) iters += (hi - lo + R - 1) / R;
  }

  WaveLane<P> wl;
  const bool odd = (lane & 1) != 0;
  bool own_in[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = kWaveCols * p + 2048 * h + 32 * lane;
      const bool in = c < K;
      wl.pk[p][h] = in ? static_cast<uint32_t>(c >> 1) : kFar;
      wl.x[p][h] = in ? static_cast<uint32_t>(c * 2) : kFar;
    }
    // the block this lane finishes: first load's (even) or second load's (odd)
    const int c0 = kWaveCols * p + (odd ? 2048 : 0) + 32 * (lane & ~1);
    own_in[p] = REG || c0 < K;  // REG: K is a multiple of 4096
    wl.c0[p] = static_cast<uint32_t>(c0);
    const uint32_t lb = static_cast<uint32_t>(c0) >> log2bs;  // its block inside the row
    wl.sq[p] = lb * (FMT == kFmtAbsmax32 ? 4u : FMT == kFmtInt4 ? 2u : 1u);
    wl.sa2[p] = FMT == kFmtInt4 ? lb * 2u : (lb >> log2s2) * 2u;
  }

  auto advance = [&](int* m_out, int* rl_out) {
    if constexpr (DYN)
      return next_group_dyn<R>(cur_c, r_end, claim, sr, C, log2C, rbeg, count, lane, m_out,
                               rl_out);
    else
      return next_group<R>(cur_c, r_end, rbeg, count, m_out, rl_out);
  };

  // the first two groups
  int m0, rl0, m1, rl1;
  int len0 = advance(&m0, &rl0);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  const nf4_gemv_desc d0 = open_desc<FMT>(descs, single, m0, len0, rbeg, K);
  int len1 = advance(&m1, &rl1);
  m1 = __builtin_amdgcn_readfirstlane(m1);
  LoadBufs lb0 = load_bufs<FMT>(d0, K, log2bs, log2s2);
  OutBufs ob0 = out_bufs<B>(d0);
  WaveGroup<R, P, FMT> g0, g1, g2;
  load_wave_group<R, P, FMT, REG>(g0, lb0, rl0, len0, wl, K, log2bs, log2s2);
  u32x4 xr[B][P][8];
  load_wave_x<B, P>(xr, x_buf<B>(d0, K), wl, K);
  float xs[B][P];  // INT4: the lane's activation sums per pass
  const void* x_cur = d0.x;  // activations held in xr
  int mL = m0;
  LoadBufs lbL = lb0;
  OutBufs ob1 = ob0;
  if (len1 > 0 && m1 != m0) {
    const nf4_gemv_desc d1 = open_desc<FMT>(descs, single, m1, len1, rbeg, K);
    lbL = load_bufs<FMT>(d1, K, log2bs, log2s2);
    ob1 = out_bufs<B>(d1);
    mL = m1;
  }
  load_wave_group<R, P, FMT, REG>(g1, lbL, rl1, len1, wl, K, log2bs, log2s2);

  if (FMT == kFmtDouble && tid < 256) s_code2[tid] = f16_to_f32(code2_bits);
  const uint32_t copy_off = build_decode_table<FMT>(s_pairs, tid, blockDim.x, lane);
  auto sum_x = [&]() {
    if constexpr (FMT == kFmtInt4) {
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          // over the 64 columns of the lane's block: the lane's half of each
          // load completed across the lane pair, as for the products
          float hs[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t w[16];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) w[4 * j + i] = xr[b][p][4 * h + j][i];
            hs[h] = pair_lane_sum(pair_sum(w));
          }
          xs[b][p] = odd ? hs[1] : hs[0];
        }
    }
  };
  sum_x();
  __syncthreads();

  auto step = [&](WaveGroup<R, P, FMT>& cur, WaveGroup<R, P, FMT>& fut) {
    int m2, rl2;
    const int len2 = advance(&m2, &rl2);
    m2 = __builtin_amdgcn_readfirstlane(m2);
    OutBufs ob2 = ob1;
    if (len2 > 0 && m2 != mL) {
      const nf4_gemv_desc d2 = open_desc<FMT>(descs, single, m2, len2, rbeg, K);
      lbL = load_bufs<FMT>(d2, K, log2bs, log2s2);
      ob2 = out_bufs<B>(d2);
      mL = m2;
    }
    load_wave_group<R, P, FMT, REG>(fut, lbL, rl2, len2, wl, K, log2bs, log2s2);
    __builtin_amdgcn_sched_barrier(0);

    // (a chunked range may end inside a round: empty groups skip the work)
    if (len0 > 0) {
      float val[R * B];
      wave_rows<B, R, P, FMT>(cur, xr, copy_off, s_pairs, s_code2, ob0.offset, odd, own_in, xs,
                              val);
      // value v of the group ends up in lane 32 v (pair) or in row 16-lane
      // row r with v = 2 (r & 1) + (r >> 1) (quad)
      float tot;
      int v;
      bool first;
      if constexpr (R * B <= 2) {
        tot = wave_sum_pair(val[0], R * B > 1 ? val[R * B - 1] : 0.0f);
        v = lane >> 5;
        first = (lane & 31) == 0;
      } else {
        tot = wave_sum_quad(val[0], val[1], val[2], R * B > 3 ? val[3] : 0.0f);
        const int row16 = lane >> 4;
        v = ((row16 & 1) << 1) | (row16 >> 1);
        first = (lane & 15) == 0;
      }
      const int rr = v / B, b = v % B;
      const bool store = first && v < R * B && rr < len0;
      const uint32_t off = static_cast<uint32_t>((b * ob0.N + rl0 + rr) * 2);
      __builtin_amdgcn_raw_buffer_store_b16(to_half_bits<NF4_BF16>(tot), ob0.y,
                                            store ? off : kOutOfRange, 0, 0);
    }
    // the next group starts a matrix with other activations: fetch them now
    // that the current ones are no longer needed
    if (len1 > 0 && m1 != m0) {
      const nf4_gemv_desc d1 = open_desc<FMT>(descs, single, m1, len1, rbeg, K);
      if (d1.x != x_cur) {
        load_wave_x<B, P>(xr, x_buf<B>(d1, K), wl, K);
        x_cur = d1.x;
        __builtin_amdgcn_s_waitcnt(0);  // rare; keeps these loads off the common path's counts
        sum_x();
      }
    }
    ob0 = ob1;
    ob1 = ob2;
    m0 = len1 > 0 ? m1 : m0;
    m1 = len2 > 0 ? m2 : m1;
    rl0 = rl1;
    rl1 = rl2;
    len0 = len1;
    len1 = len2;
  };
  // Whole rounds of three steps (see gemv_stream_kernel for why no step ends
  // the loop); with DYN the number of groups is not known in advance, and
  // the at most two empty steps of the last round skip their work.
  const int slot = static_cast<int>(__builtin_amdgcn_s_getreg(kHwRegWaveSlot));
  if constexpr (DYN) {
    for (int it = 0; len0 > 0; ++it) {
      rotate_priority(it, slot);
      step(g0, g2);
      step(g1, g0);
      step(g2, g1);
    }
    // the last wave of the region returns its counters to zero, so the
    // workspace is ready for the next launch: every claim of this launch has
    // returned by now (each wave read its last one before stopping)
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) {
      const unsigned prev = atomicAdd(sr.done, 1u);
      if (prev == static_cast<unsigned>(sr.W - 1)) {
        atomicExch(sr.claims, 0u);
        atomicExch(sr.done, 0u);
      }
    }
  } else {
    const int rounds = iters / 3;
    for (int it = 0; it < rounds; ++it) {
      rotate_priority(it, slot);
      step(g0, g2);
      step(g1, g0);
      step(g2, g1);
    }
    const int rest = iters - 3 * rounds;
    if (rest > 0) step(g0, g2);
    if (rest > 1) step(g1, g0);
  }
}

// One pass (4096 columns) of R rows for one lane, with the activations read
// from the workgroup's LDS copy: s_xp points at the lane's entry of dword 0 of
// the pass for batch row 0, and batch row b is bstride entries further.  The
// lane's eight packed dwords per row (two loads of four) are walked in order,
// rows inner: the B activation quads of a dword are read once and serve all R
// rows, and the table entries of the next (dword, row) are read before the
// current one's products.  At the end of each load the two half sums of a
// block are completed across the lane pair and the lane scales the block it
// owns (odd lanes: the second load's).  val is assigned when `first` (the
// row's first pass), accumulated otherwise.
template <int B, int R, int FMT>
__device__ __forceinline__ void xpass_rows(const WaveGroup<R, 1, FMT>& g, uint32_t copy_off,
                                           const uint2* s_pairs, const float* s_code2,
                                           float offset, bool odd, bool own_in,
                                           const float (&xs)[B], float (&val)[R * B], bool first,
                                           const u32x4* s_xp, int bstride) {
  constexpr int U = 8 * R;
  const char* tab = reinterpret_cast<const char*>(s_pairs);
  uint2 t[2][4];
  u32x4 xv[2][B];
  auto fetch = [&](int u, uint2 (&tt)[4]) {
    const int hj = u / R, rr = u % R;
    const uint32_t d = g.pk[rr][0][hj >> 2][hj & 3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t addr = __builtin_amdgcn_perm(copy_off, d, 0x0C0C0004u | (uint32_t(i) << 8));
      if constexpr (FMT == kFmtInt4)
        tt[i].x = *reinterpret_cast<const uint32_t*>(tab + addr);  // one exact code pair
      else
        tt[i] = *reinterpret_cast<const uint2*>(tab + addr);
    }
    if (rr == 0) {
#pragma unroll
      for (int b = 0; b < B; ++b) xv[hj & 1][b] = s_xp[b * bstride + hj * 64];
    }
  };
  float part[R][B], half0[R][B];
  fetch(0, t[0]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u + 1 < U) fetch(u + 1, t[(u + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    const int hj = u / R, rr = u % R;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 ti = t[u & 1][i];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        // copied out first: a bit_cast of a vector-element lvalue reads
        // element 0 whatever the index
        const uint32_t xw = xv[hj & 1][b][i];
        const bf16x2 xp = __builtin_bit_cast(bf16x2, xw);
        // the first product of each half starts from an immediate zero
        const float acc = (hj & 3) == 0 && i == 0 ? 0.0f : part[rr][b];
        part[rr][b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ti.x), xp, acc,
                                                      false);
        if constexpr (FMT != kFmtInt4)
          part[rr][b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ti.y), xp,
                                                        part[rr][b], false);
      }
    }
    if (hj == 3) {
#pragma unroll
      for (int b = 0; b < B; ++b) half0[rr][b] = part[rr][b];
    }
    if (hj == 7) {
      float blk[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float s0 = pair_lane_sum(half0[rr][b]);
        const float s1 = pair_lane_sum(part[rr][b]);
        blk[b] = odd ? s1 : s0;
      }
      if constexpr (FMT == kFmtInt4) {
        const float sc = f16_to_f32(g.q[rr][0]);
        const float z = f16_to_f32(g.a2[rr][0]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float zt = z * xs[b];
          const float c = own_in ? sc * (blk[b] - zt) : 0.0f;
          val[rr * B + b] = first ? c : val[rr * B + b] + c;
        }
      } else {
        float a;
        if constexpr (FMT == kFmtAbsmax32) {
          a = __builtin_bit_cast(float, g.q[rr][0]);
        } else {
          const float prod = s_code2[g.q[rr][0]] * f16_to_f32(g.a2[rr][0]);
          a = prod + offset;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float c = own_in ? a * blk[b] : 0.0f;
          val[rr * B + b] = first ? c : val[rr * B + b] + c;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// The shared-activation GEMV (grouped launches, K % 64 == 0, blocksize >= 64:
// batch 1-2 with 4096 < K <= 16384, and batch 3-8 with K <= 4096).
//
// With more than one pass the wave kernel keeps 32 B P VGPRs of activations
// per wave and fits only two waves per SIMD: too few independent instruction
// streams to keep the VALU and LDS busy.  Here a 1024-thread workgroup (16
// waves, four per SIMD, one workgroup per CU) keeps the activations of the
// matrix it works on in LDS, in the lane order in which the wave kernel holds
// them in registers, so each ds_read_b128 of the 64 lanes reads 1 KiB of
// consecutive banks.  The lane layout, decode and per-row arithmetic are the
// wave kernel's (wave_rows with XL).  At batch 3-8 the activations of every
// batch row are in LDS (8 KiB each) and a wave computes one row per group.
//
// The concatenated rows are split evenly into one contiguous range per
// workgroup.  The workgroup walks its range one matrix at a time: it stages
// that matrix's activations (a barrier before and after), then its waves
// claim groups of R rows from an LDS counter until the matrix's part of the
// range is used up.  A wave's unit of work is one pass of its R rows: for
// every packed dword it reads the activations once and applies them to all R
// rows, so the activation reads from LDS per weight byte fall by R (the LDS
// bandwidth, shared by the decode table reads, bounds this kernel).  Each wave
// keeps NB register buffers of units, NB a multiple of P, so that buffer j
// always holds pass j % P: the loads of the unit NB - 1 ahead are issued
// before the current unit is computed, and a new row group is claimed when
// its first pass is loaded.  The loops run whole rounds of NB units.
// ---------------------------------------------------------------------------
constexpr int kXlThreads = 1024;

template <int B, int R, int P, int NB, int FMT>
__global__ __launch_bounds__(kXlThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemv_xlds_kernel(
    const nf4_gemv_desc* __restrict__ descs, int count, int total_rows, int K, int log2bs,
    int log2s2, const uint16_t* __restrict__ code2) {
  static_assert(R * B <= 8, "at most two quad reductions per group");
  static_assert(NB >= 2 && NB % P == 0, "whole passes per round, at least two buffers");
  __shared__ uint2 s_pairs[256 * kPairCopies];  // 64 KiB decode table
  __shared__ float s_code2[256];
  __shared__ int s_rowbeg[kMaxDescs + 1];
  __shared__ u32x4 s_x[B * P * 8 * 64];  // activations, 8 KiB per pass and batch row
  __shared__ unsigned s_next;            // next row group of the current matrix
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint16_t code2_bits = __builtin_amdgcn_raw_buffer_load_b16(
      rsrc(FMT == kFmtDouble ? code2 : nullptr, 512), static_cast<uint32_t>(tid) * 2u, 0u, 0);
  for (int i = tid; i < count; i += blockDim.x) s_rowbeg[i] = static_cast<int>(descs[i].row_begin);
  if (tid == 0) s_rowbeg[count] = total_rows;
  if (FMT == kFmtDouble && tid < 256) s_code2[tid] = f16_to_f32(code2_bits);
  const uint32_t copy_off = build_decode_table<FMT>(s_pairs, tid, blockDim.x, lane);
  __syncthreads();
  const RowBegins rbeg{s_rowbeg, total_rows};
  int lo, hi;
  split_rows(static_cast<uint32_t>(total_rows), gridDim.x, blockIdx.x, &lo, &hi);

  // the lane's columns, as in the wave kernel
  WaveLane<P> wl;
  const bool odd = (lane & 1) != 0;
  bool own_in[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = kWaveCols * p + 2048 * h + 32 * lane;
      wl.pk[p][h] = c < K ? static_cast<uint32_t>(c >> 1) : kFar;
      wl.x[p][h] = kFar;  // activations come from LDS
    }
    const int c0 = kWaveCols * p + (odd ? 2048 : 0) + 32 * (lane & ~1);
    own_in[p] = c0 < K;
    wl.c0[p] = static_cast<uint32_t>(c0);
  }

  int m = 0;  // last matrix whose first row is <= lo
  {
    int a = 0, z = count - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (rbeg(mid) <= lo) a = mid; else z = mid - 1;
    }
    m = a;
  }
  for (; m < count && rbeg(m) < hi; ++m) {
    const int beg = rbeg(m), end = rbeg(m + 1);
    const int s0 = max(lo, beg), s1 = min(hi, end);
    if (s1 <= s0) continue;
    const nf4_gemv_desc d = open_desc<FMT>(descs, nf4_gemv_desc{}, m, s1 - s0, rbeg, K);
    __syncthreads();  // every wave is done with the previous matrix's activations
    {
      // entry e = ((b P + p) 8 + hj) 64 + l: columns 4096 p + 2048 (hj >> 2) +
      // 32 l + 8 (hj & 3), 8 of them, of batch row b (zeros past K)
      const __amdgpu_buffer_rsrc_t xb = rsrc(d.x, static_cast<uint32_t>(B * K * 2));
      for (int e = tid; e < B * P * 8 * 64; e += kXlThreads) {
        const int l = e & 63, hj = (e >> 6) & 7, bp = e >> 9;
        const int b = bp / P, p = bp - b * P;
        const int c = kWaveCols * p + 2048 * (hj >> 2) + 32 * l + 8 * (hj & 3);
        s_x[e] = __builtin_amdgcn_raw_buffer_load_b128(
            xb, c < K ? static_cast<uint32_t>((b * K + c) * 2) : kFar, 0u, 0);
      }
    }
    if (tid == 0) s_next = 0;
    __syncthreads();
    if (d.packed == nullptr) continue;  // a skipped matrix (the same for every wave)
    const LoadBufs lb = load_bufs<FMT>(d, K, log2bs, log2s2);
    const OutBufs ob = out_bufs<B>(d);
    float xs[B][P];  // INT4: the activation sums of the lane's blocks
    if constexpr (FMT == kFmtInt4) {
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          float hs[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t w[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 q = s_x[((b * P + p) * 8 + 4 * h + j) * 64 + lane];
#pragma unroll
              for (int i = 0; i < 4; ++i) w[4 * j + i] = q[i];
            }
            hs[h] = pair_lane_sum(pair_sum(w));
          }
          xs[b][p] = odd ? hs[1] : hs[0];
        }
    }
    const int base = s0 - beg;  // first row of this part, inside the matrix
    const int nrows = s1 - s0;
    auto claim = [&](int* rl, int* len) {
      uint32_t g = 0;
      if (lane == 0) g = atomicAdd(&s_next, 1u);
      g = __builtin_amdgcn_readfirstlane(g);
      const int r = static_cast<int>(g) * R;
      *rl = base + r;
      *len = r < nrows ? min(R, nrows - r) : 0;
    };
    // the group's rows and y: reduce the R B row values over the lanes and
    // store them
    auto finish = [&](const float (&val)[R * B], int rl, int len) {
      // one pair or quad reduction per four values
      constexpr int NQ = R * B <= 4 ? 1 : 2;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        float tot;
        int v;
        bool first;
        if constexpr (R * B <= 2) {
          tot = wave_sum_pair(val[0], R * B > 1 ? val[R * B - 1] : 0.0f);
          v = lane >> 5;
          first = (lane & 31) == 0;
        } else {
          const int o = 4 * qd;
          tot = wave_sum_quad(val[o], o + 1 < R * B ? val[o + 1] : 0.0f,
                              o + 2 < R * B ? val[o + 2] : 0.0f,
                              o + 3 < R * B ? val[o + 3] : 0.0f);
          const int row16 = lane >> 4;
          v = o + (((row16 & 1) << 1) | (row16 >> 1));
          first = (lane & 15) == 0;
        }
        const int rr = v / B, b = v % B;
        const bool store = first && v < R * B && rr < len;
        const uint32_t off = static_cast<uint32_t>((b * ob.N + rl + rr) * 2);
        __builtin_amdgcn_raw_buffer_store_b16(to_half_bits<NF4_BF16>(tot), ob.y,
                                              store ? off : kOutOfRange, 0, 0);
      }
    };
    // the lane's columns of pass q as a one-pass lane description
    auto pass_lane = [&](int q) {
      WaveLane<1> w1;
      w1.pk[0][0] = wl.pk[q][0];
      w1.pk[0][1] = wl.pk[q][1];
      w1.x[0][0] = w1.x[0][1] = kFar;
      w1.c0[0] = wl.c0[q];
      w1.sq[0] = w1.sa2[0] = 0u;
      return w1;
    };
    WaveGroup<R, 1, FMT> gb[NB];
    int rlb[NB], lenb[NB];
    int crl = 0, clen = 0;  // the row group claimed last
    // prologue: the first NB - 1 units
#pragma unroll
    for (int j = 0; j + 1 < NB; ++j) {
      if (j % P == 0) claim(&crl, &clen);
      rlb[j] = crl;
      lenb[j] = clen;
      load_wave_group<R, 1, FMT>(gb[j], lb, crl, clen, pass_lane(j % P), K, log2bs, log2s2);
    }
    float val[R * B];
    while (lenb[0] > 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        // the unit NB - 1 ahead goes into the buffer computed last
        const int f = (j + NB - 1) % NB;
        if (f % P == 0) claim(&crl, &clen);
        rlb[f] = crl;
        lenb[f] = clen;
        load_wave_group<R, 1, FMT>(gb[f], lb, crl, clen, pass_lane(f % P), K, log2bs, log2s2);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int kPassEntries = 8 * 64;
        const int q = j % P;
        if (lenb[j] > 0) {
          float xsq[B];
#pragma unroll
          for (int bb = 0; bb < B; ++bb) xsq[bb] = xs[bb][q];
          xpass_rows<B, R, FMT>(gb[j], copy_off, s_pairs, s_code2, ob.offset, odd, own_in[q], xsq,
                                val, q == 0, s_x + q * kPassEntries + lane, P * kPassEntries);
          if (q == P - 1) finish(val, rlb[j], lenb[j]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused dequant-GEMV, batched path (batch 3-8).
//
// A workgroup owns R consecutive rows and has one wave per 2048-column slab
// of K (W = ceil(K / 2048) waves, at most 8).  Lane l of wave s covers the 32
// columns [2048 s + 32 l, +32): one 16-byte packed load per row, lying inside
// one first-level block (blocksize >= 32, K % 32 == 0), so the lane computes
// one absmax_real per row and applies it after summing its 32 products
// (scale after accumulate).  The lane's 32 activations per batch row are
// loaded once and reused for all R rows.  Lane partials are reduced with DPP,
// the W wave partials in LDS in a fixed order; one bf16 store per output.
// Requirements (checked on the host): K % 32 == 0, K <= 16384, blocksize >=
// 32, packed 16-byte aligned, x 16-byte aligned.
// ---------------------------------------------------------------------------
template <int B, int R, int FMT = kFmtDouble>
__global__ __launch_bounds__(512) void gemv_vec_kernel(
    const uint4* __restrict__ packed16, const uint8_t* __restrict__ absmax_q,
    const uint16_t* __restrict__ absmax2, const uint16_t* __restrict__ code2, float offset,
    int N, int K, int log2bs, int log2s2, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y) {
  __shared__ float s_nf4[16];
  __shared__ float s_code2[256];
  __shared__ float s_red[8][R * B];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int r0 = blockIdx.x * R;
  const int k0 = wave * kSlab + lane * 32;
  const bool active = k0 < K;

  uint4 pk[R];
  uint32_t qv[R];
  float a2v[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int r = r0 + rr;
    if (active && r < N) {
      const int64_t e = static_cast<int64_t>(r) * K + k0;
      const int64_t blk = e >> log2bs;
      pk[rr] = packed16[e >> 5];
      if constexpr (FMT == kFmtAbsmax32) {
        qv[rr] = reinterpret_cast<const uint32_t*>(absmax_q)[blk];
        a2v[rr] = 0.0f;
      } else if constexpr (FMT == kFmtInt4) {
        qv[rr] = reinterpret_cast<const uint16_t*>(absmax_q)[blk];  // scale
        a2v[rr] = f16_to_f32(absmax2[blk]);                          // zero point
      } else {
        qv[rr] = absmax_q[blk];
        a2v[rr] = f16_to_f32(absmax2[blk >> log2s2]);
      }
    } else {
      pk[rr] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
      qv[rr] = 0;
      a2v[rr] = 0.0f;
    }
  }
  if constexpr (FMT == kFmtDouble)
    for (int i = threadIdx.x; i < 256; i += blockDim.x) s_code2[i] = f16_to_f32(code2[i]);
  if (threadIdx.x < 16) s_nf4[threadIdx.x] = code_value<FMT>(threadIdx.x);
  __syncthreads();
  float a[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if constexpr (FMT == kFmtAbsmax32) {
      a[rr] = __builtin_bit_cast(float, qv[rr]);
    } else if constexpr (FMT == kFmtInt4) {
      a[rr] = f16_to_f32(static_cast<uint16_t>(qv[rr]));
    } else {
      const float prod = s_code2[qv[rr]] * a2v[rr];
      a[rr] = prod + offset;
    }
  }

  float part[R][B];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int b = 0; b < B; ++b) part[rr][b] = 0.0f;

#pragma unroll
  for (int j = 0; j < 4; ++j) {  // 8 columns per sub-step
    uint32_t xw[B][4];            // raw bf16 pairs of the 8 columns
#pragma unroll
    for (int b = 0; b < B; ++b) {
      uint4 xr = make_uint4(0u, 0u, 0u, 0u);
      if (active) xr = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(b) * K + k0 + 8 * j);
      xw[b][0] = xr.x;
      xw[b][1] = xr.y;
      xw[b][2] = xr.z;
      xw[b][3] = xr.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // one packed byte = two columns
      float xe[B], xo[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xe[b] = __builtin_bit_cast(float, xw[b][i] << 16);
        xo[b] = __builtin_bit_cast(float, xw[b][i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const uint32_t wd = j == 0 ? pk[rr].x : j == 1 ? pk[rr].y : j == 2 ? pk[rr].z : pk[rr].w;
        float te, to;
        if constexpr (FMT == kFmtInt4) {  // (q - z), exact; the scale comes after the sum
          te = s_nf4[(wd >> (8 * i)) & 15u] - a2v[rr];
          to = s_nf4[(wd >> (8 * i + 4)) & 15u] - a2v[rr];
        } else {
          te = s_nf4[(wd >> (8 * i + 4)) & 15u];
          to = s_nf4[(wd >> (8 * i)) & 15u];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          part[rr][b] = __builtin_fmaf(te, xe[b], part[rr][b]);
          part[rr][b] = __builtin_fmaf(to, xo[b], part[rr][b]);
        }
      }
    }
  }

#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float tot = wave_sum_to_lane63(a[rr] * part[rr][b]);
      if (lane == 63) s_red[wave][rr * B + b] = tot;
    }
  __syncthreads();
  if (threadIdx.x < R * B) {
    const int rr = threadIdx.x / B, b = threadIdx.x % B;
    float acc = s_red[0][threadIdx.x];
    for (int w = 1; w < nwaves; ++w) acc += s_red[w][threadIdx.x];
    const int r = r0 + rr;
    if (r < N) y[static_cast<int64_t>(b) * N + r] = to_half_bits<NF4_BF16>(acc);
  }
}

// ---------------------------------------------------------------------------
// Fused dequant-GEMV, general path: one wave per row, lanes stride over the
// row two elements (one byte) at a time, per-element scales.  Any even K,
// any power-of-two block sizes, any alignment.
// ---------------------------------------------------------------------------
template <int B, int FMT = kFmtDouble>
__global__ __launch_bounds__(256) void gemv_any_kernel(
    const uint8_t* __restrict__ packed8, const uint8_t* __restrict__ absmax_q,
    const uint16_t* __restrict__ absmax2, const uint16_t* __restrict__ code2, float offset,
    int64_t N, int64_t K, int log2bs, int log2s2, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y) {
  __shared__ float s_nf4[16];
  if (threadIdx.x < 16) s_nf4[threadIdx.x] = code_value<FMT>(threadIdx.x);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (r >= N) return;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  for (int64_t k = 2 * lane; k < K; k += 128) {
    const int64_t e = r * K + k;
    const uint8_t byte = packed8[e >> 1];
    const float ve = element_value<FMT>(s_nf4, nibble_of<FMT>(byte, 0), absmax_q, absmax2, code2,
                                        offset, e >> log2bs, log2s2);
    const float vo = element_value<FMT>(s_nf4, nibble_of<FMT>(byte, 1), absmax_q, absmax2, code2,
                                        offset, (e + 1) >> log2bs, log2s2);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float x0 = __builtin_bit_cast(float, static_cast<uint32_t>(x[b * K + k]) << 16);
      const float x1 = __builtin_bit_cast(float, static_cast<uint32_t>(x[b * K + k + 1]) << 16);
      acc[b] = __builtin_fmaf(ve, x0, acc[b]);
      acc[b] = __builtin_fmaf(vo, x1, acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float tot = wave_sum_to_lane63(acc[b]);
    if (lane == 63) y[b * N + r] = to_half_bits<NF4_BF16>(tot);
  }
}

// y = 0 for an empty reduction (K == 0).
// Zeroes a scheduling workspace of `count` counters (one small workgroup).
__global__ void sched_clear_kernel(unsigned* __restrict__ sched, int count) {
  for (int i = threadIdx.x; i < count; i += blockDim.x) sched[i] = 0u;
}

__global__ void fill_zero_kernel(uint16_t* __restrict__ y, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += stride)
    y[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool pow2_log2(int32_t v, int* lg) {
  if (v < 1 || v > (1 << 30) || (v & (v - 1)) != 0) return false;
  int l = 0;
  while ((1 << l) < v) ++l;
  *lg = l;
  return true;
}

template <int OUT, int FMT>
nf4_status dequant_launch(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                          const uint16_t* code2, float offset, int64_t n, int lbs, int ls2,
                          void* out, hipStream_t st) {
  const bool vec = lbs >= 3 && aligned(packed, 4) && aligned(out, 16);
  if (vec) {
    const int64_t steps = (n >> 3) + ((n & 7) ? 1 : 0);
    const int64_t cus = device_cus();
    const int U = steps >= cus * kDqThreads * 4 ? 4 : (steps >= cus * kDqThreads * 2 ? 2 : 1);
    const int64_t tiles = (steps + kDqThreads * U - 1) / (kDqThreads * U);
    if (tiles > 0x7FFFFFFF) return NF4_EUNSUPPORTED;
    const auto kernel = U == 4   ? dequant_vec_kernel<OUT, 4, FMT>
                        : U == 2 ? dequant_vec_kernel<OUT, 2, FMT>
                                 : dequant_vec_kernel<OUT, 1, FMT>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(tiles)), dim3(kDqThreads), 0, st,
                       reinterpret_cast<const uint32_t*>(packed), packed, absmax_q, absmax2, code2,
                       offset, n, lbs, ls2, reinterpret_cast<u32x4*>(out),
                       reinterpret_cast<uint16_t*>(out));
  } else {
    const int64_t blocks = (n + 255) / 256;
    const uint32_t grid = static_cast<uint32_t>(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL((dequant_any_kernel<OUT, FMT>), dim3(grid), dim3(256), 0, st, packed, absmax_q,
                       absmax2, code2, offset, n, lbs, ls2, reinterpret_cast<uint16_t*>(out));
  }
  return launch_status();
}

// rows per group: 4 at batch 1, 2 at batch 2 (four values per wave
// reduction; with prefetch depth 2 this stays within the 128 VGPRs of four
// waves per SIMD), 1 at batch 3-4, 2 at batch 5-8 (half the reductions and
// barriers per row; 192-249 VGPRs, within the two waves per SIMD these
// batches run at).  Waves per SIMD: the activations take 16 B VGPRs, so
// batches above 4 run at two waves per SIMD (one workgroup per CU).
template <int B>
constexpr int stream_rows() { return B == 1 ? 4 : (B == 2 ? 2 : (B >= 5 ? 2 : 1)); }
template <int B>
constexpr int stream_wpe() { return B <= 4 ? 4 : 2; }

template <int B, int NW, int FMT>
void stream_launch_nw(const nf4_gemv_desc* descs, const nf4_gemv_desc& single, int count,
                      int total_rows, int K, int lbs, int ls2, const uint16_t* code2,
                      int64_t grid, hipStream_t st) {
  if (descs == nullptr)
    hipLaunchKernelGGL((gemv_stream_kernel<B, stream_rows<B>(), NW, stream_wpe<B>(), FMT, true>),
                       dim3(static_cast<uint32_t>(grid)), dim3(512), 0, st, descs, single, 1,
                       total_rows, K, lbs, ls2, code2);
  else
    hipLaunchKernelGGL((gemv_stream_kernel<B, stream_rows<B>(), NW, stream_wpe<B>(), FMT>),
                       dim3(static_cast<uint32_t>(grid)), dim3(512), 0, st, descs, single, count,
                       total_rows, K, lbs, ls2, code2);
}

// Rows of the contiguous static share each wave takes before it claims
// chunks of C: three quarters of its even share, rounded down to whole chunks
// (at least one).  Every claim costs the claiming wave: the atomic's reply
// returns in order with the wave's loads, and under a full memory stream it
// holds up the loads issued after it.  With the rotating wave priority the
// waves progress nearly evenly through their static shares, so the chunked
// quarter is enough to even out the rest.  Measured on the 192-matrix K = 4096
// sweep launch (three runs each): 1/2 static share without rotation 430 us,
// with rotation 1/2 -> 421, 2/3 -> 421, 3/4 -> 418, 7/8 -> 429; the same
// launch with the loads alone and a static split streams in 385 us.
inline int dyn_static_rows(int64_t rows_per_wave, int C) {
  const int64_t s = rows_per_wave * 3 / 4 / C * C;
  return s > C ? static_cast<int>(s) : C;
}

// The wave-per-row kernel for (B, P): rows per group and waves per SIMD are
// set by registers: the activations take 32 B P VGPRs, each row group 10 R P,
// and three groups are in flight.  With a scheduling workspace, four waves per
// SIMD and at least 64 rows per wave, rows are handed out in chunks (see
// SchedRegion): about 16 chunks per wave, 4 to 32 rows each.
template <int B, int R, int P, int WPE, int FMT>
nf4_status wave_launch(const nf4_gemv_desc* descs, const nf4_gemv_desc& single, int count,
                       int total_rows, int K, int lbs, int ls2, const uint16_t* code2,
                       unsigned* sched, bool sched_clear, hipStream_t st) {
  // One row per wave at most one 512-lane workgroup per CU; a second one per
  // CU (four waves per SIMD) only once every wave gets two rows or more: with
  // one row per wave the younger workgroup mostly waits behind the older one
  // (4096 x 4096 takes 9.4 us on two per CU, 7.3 us on one).
  const int64_t cus = device_cus();
  const int64_t want = (static_cast<int64_t>(total_rows) + 7) / 8;
  int64_t grid = want < cus ? (want > 0 ? want : 1) : cus;
  if (WPE == 4 && want >= 4 * cus) grid = want < 2 * cus ? want : 2 * cus;
  const int64_t rows_per_wave = (static_cast<int64_t>(total_rows) + grid * 8 - 1) / (grid * 8);
  const bool dyn = WPE == 4 && sched != nullptr && rows_per_wave >= 64;
  int C = 0, S = 0;
  if (dyn) {
    C = 4;
    while (C < 32 && C * 2 * 16 <= rows_per_wave) C *= 2;
    S = dyn_static_rows(rows_per_wave, C);
  }
  // regular shapes (see load_wave_group): whole 4096-column passes, whole
  // blocks per row, and blocks per row and s2 dividing one into the other
  const int64_t bs = int64_t(1) << lbs, s2 = int64_t(1) << ls2;
  const int64_t nb = K / bs;  // blocks per row when K % bs == 0
  const bool reg = K % kWaveCols == 0 && K % bs == 0 &&
                   (FMT != kFmtDouble || nb % s2 == 0 || s2 % nb == 0);
  const dim3 g(static_cast<uint32_t>(grid)), blk(512);
  unsigned* sc = dyn ? sched : nullptr;
  // a workspace whose contents are not known to be zero (the library's own
  // scratch) is cleared by a kernel on the same stream first
  if (dyn && sched_clear)
    hipLaunchKernelGGL(sched_clear_kernel, dim3(1), dim3(256), 0, st, sched,
                       kSchedRegions * kSchedStride);
  if (reg && dyn)
    hipLaunchKernelGGL((gemv_wave_kernel<B, R, P, WPE, true, FMT, true>), g, blk, 0, st, descs,
                       single, count, total_rows, K, lbs, ls2, code2, sc, C, S);
  else if (reg)
    hipLaunchKernelGGL((gemv_wave_kernel<B, R, P, WPE, false, FMT, true>), g, blk, 0, st, descs,
                       single, count, total_rows, K, lbs, ls2, code2, sc, C, S);
  else if (dyn)
    hipLaunchKernelGGL((gemv_wave_kernel<B, R, P, WPE, true, FMT, false>), g, blk, 0, st, descs,
                       single, count, total_rows, K, lbs, ls2, code2, sc, C, S);
  else
    hipLaunchKernelGGL((gemv_wave_kernel<B, R, P, WPE, false, FMT, false>), g, blk, 0, st,
                       descs, single, count, total_rows, K, lbs, ls2, code2, sc, C, S);
  return launch_status();
}

// Whether a grouped launch has rows enough for the shared-activation kernel:
// at least two per wave of a full grid.  With fewer its waves have nothing to
// pipeline and the team kernel, which splits each row over several waves, is
// faster (one 4096 x 11008 matrix: 20.8 us against 12.8; two: 21.9 against
// 23.0; four: 28.2 against 45.1).
inline bool xlds_rows_ok(int total_rows) {
  return static_cast<int64_t>(total_rows) >= 2 * (kXlThreads / 64) * device_cus();
}

// The shared-activation kernel for (B, P): one 1024-thread workgroup per CU
// at most, each with at least 64 rows.
template <int B, int R, int P, int NB, int FMT>
nf4_status xlds_launch(const nf4_gemv_desc* descs, int count, int total_rows, int K, int lbs,
                       int ls2, const uint16_t* code2, hipStream_t st) {
  const int64_t cus = device_cus();
  const int64_t want = (static_cast<int64_t>(total_rows) + 63) / 64;
  const int64_t grid = want < cus ? (want > 0 ? want : 1) : cus;
  hipLaunchKernelGGL((gemv_xlds_kernel<B, R, P, NB, FMT>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kXlThreads), 0, st, descs, count, total_rows, K, lbs, ls2, code2);
  return launch_status();
}

// Returns NF4_EUNSUPPORTED (without launching) when no wave-per-row
// configuration covers (B, K, blocksize).
template <int B, int FMT>
nf4_status wave_dispatch(const nf4_gemv_desc* descs, const nf4_gemv_desc& single, int count,
                         int total_rows, int K, int lbs, int ls2, const uint16_t* code2,
                         unsigned* sched, bool sched_clear, hipStream_t st) {
  if (K % 64 != 0 || lbs < 6) return NF4_EUNSUPPORTED;
  const int P = (K + kWaveCols - 1) / kWaveCols;
  if constexpr (B == 1) {
    if (P == 1) return wave_launch<1, 2, 1, 4, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, sched, sched_clear, st);
  }
  // the other configurations serve grouped launches only
  if constexpr (B == 2) {
    if (P == 1) return wave_launch<2, 1, 1, 4, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, sched, sched_clear, st);
  }
  // more than one pass: the activations go to LDS (gemv_xlds_kernel), for
  // launches that give every wave two rows or more (see xlds_rows_ok)
  if (descs == nullptr || !xlds_rows_ok(total_rows)) return NF4_EUNSUPPORTED;
  if constexpr (B == 1) {
    if (P == 2) return xlds_launch<1, 2, 2, 4, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
    if (P == 3) return xlds_launch<1, 2, 3, 3, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
    if (P == 4) return xlds_launch<1, 1, 4, 4, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
  } else if constexpr (B == 2) {
    if (P == 2) return xlds_launch<2, 2, 2, 2, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
    if (P == 3) return xlds_launch<2, 2, 3, 3, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
    if (P == 4) return xlds_launch<2, 1, 4, 4, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
  }
  return NF4_EUNSUPPORTED;
}

template <int B, int FMT>
nf4_status stream_launch(const nf4_gemv_desc* descs, const nf4_gemv_desc& single, int count,
                         int total_rows, int K, int lbs, int ls2, const uint16_t* code2,
                         unsigned* sched, hipStream_t st, bool sched_clear = false) {
  // grouped launches at batch 3-8 with one pass: the shared-activation kernel
  // (four waves per SIMD, no barrier per row group; 16% faster than the team
  // kernel at batch 4, 3% at batch 8)
  if constexpr (B >= 3) {
    if (descs != nullptr && K % 64 == 0 && K <= kWaveCols && lbs >= 6 &&
        xlds_rows_ok(total_rows))
      return xlds_launch<B, (B <= 4 && FMT != kFmtInt4 ? 2 : 1), 1, 2, FMT>(descs, count, total_rows, K, lbs, ls2, code2, st);
  }
  // Grouped launches (descs != NULL) at batch 1-2 take the wave kernel.  A
  // single matrix takes it only at batch 1, one pass and up to 2^24 weights:
  // there every wave has one or two rows and the wave kernel's lighter
  // prologue wins (4096 x 4096: 6.8 us against 7.8).  Past that, and at batch
  // 2, a single launch has all its loads in flight almost at once and ends
  // with each wave's serial decode of its rows; the team kernel splits every
  // row over several waves and finishes sooner (11008 x 4096: 11.0 us against
  // 12.0; 4096 x 11008: 11.2 against 14.5; 4096 x 4096 at batch 2: 7.2
  // against 8.7).  In a long grouped launch the wave kernel's rows pipeline
  // and it streams faster than the team kernel.
  if constexpr (B <= 2) {
    const bool single_ok =
        B == 1 && K <= kWaveCols && static_cast<int64_t>(total_rows) * K <= (int64_t(1) << 24);
    if (descs != nullptr || single_ok) {
      const nf4_status ws =
          wave_dispatch<B, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, sched,
                                sched_clear, st);
      if (ws != NF4_EUNSUPPORTED) return ws;
    }
  }
  // one matrix at batch 3-8 with K <= 4096: fp32 products (see
  // dot_columns_f32) with 16 columns per lane, so the fp32 activations take
  // 16 B VGPRs; one row per group at batch 3-4, two at 5-8
  if constexpr (B >= 3 && FMT == kFmtDouble) {
    if (descs == nullptr && K <= 4096) {
      constexpr int RX = B <= 4 ? 1 : 2;
      constexpr int WX = B <= 4 ? 4 : 2;
      const int nwx = (K + 1023) / 1024;
      const int teams_x = 8 / nwx;
      const int64_t cap = static_cast<int64_t>(device_cus()) * (WX / 2);
      const int64_t want_x = (static_cast<int64_t>(total_rows) + teams_x * RX - 1) / (teams_x * RX);
      const int64_t gx = want_x < cap ? (want_x > 0 ? want_x : 1) : cap;
      const dim3 g(static_cast<uint32_t>(gx)), blk(512);
      switch (nwx) {
#define NF4_XF_CASE(NWX)                                                                          \
  case NWX:                                                                                       \
    hipLaunchKernelGGL((gemv_stream_kernel<B, RX, NWX, WX, FMT, true, 2, true>), g, blk, 0, st,   \
                       nullptr, single, 1, total_rows, K, lbs, ls2, code2);                       \
    break;
        NF4_XF_CASE(1)
        NF4_XF_CASE(2)
        NF4_XF_CASE(3)
        NF4_XF_CASE(4)
#undef NF4_XF_CASE
        default: return NF4_EUNSUPPORTED;
      }
      return launch_status();
    }
  }
  const int nw = (K + kSlab - 1) / kSlab;
  const int teams = 8 / nw;
  // persistent: at most two 512-lane workgroups per CU (the decode table takes
  // 64 KiB of LDS; one at two waves per SIMD), at least one row per team
  const int64_t max_wg = static_cast<int64_t>(device_cus()) * (stream_wpe<B>() / 2);
  const int64_t want = (static_cast<int64_t>(total_rows) + teams - 1) / teams;
  const int64_t grid = want < max_wg ? (want > 0 ? want : 1) : max_wg;
  switch (nw) {
    case 1: stream_launch_nw<B, 1, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 2: stream_launch_nw<B, 2, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 3: stream_launch_nw<B, 3, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 4: stream_launch_nw<B, 4, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 5: stream_launch_nw<B, 5, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 6: stream_launch_nw<B, 6, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 7: stream_launch_nw<B, 7, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    case 8: stream_launch_nw<B, 8, FMT>(descs, single, count, total_rows, K, lbs, ls2, code2, grid, st); break;
    default: return NF4_EUNSUPPORTED;
  }
  return launch_status();
}

template <int B, int FMT>
nf4_status gemv_launch_b(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                         const uint16_t* code2, float offset, int64_t N, int64_t K, int lbs,
                         int ls2, const uint16_t* x, uint16_t* y, hipStream_t st) {
  const bool vec = lbs >= 5 && K % 32 == 0 && K <= 8 * kSlab && N <= 0x7FFFFFFF &&
                   aligned(packed, 16) && aligned(x, 16);
  if (vec && N * K < (int64_t(1) << 31)) {  // the streaming kernels' offset range
    nf4_gemv_desc one{};
    one.packed = packed;
    one.absmax_q = absmax_q;
    one.absmax2 = absmax2;
    one.x = x;
    one.y = y;
    one.N = N;
    one.row_begin = 0;
    one.offset = offset;
    return stream_launch<B, FMT>(nullptr, one, 1, static_cast<int>(N), static_cast<int>(K), lbs,
                                 ls2, code2, nullptr, st);
  }
  if (vec) {
    constexpr int R = B <= 4 ? 2 : 1;
    const int nw = static_cast<int>((K + kSlab - 1) / kSlab);
    const int64_t grid = (N + R - 1) / R;
    hipLaunchKernelGGL((gemv_vec_kernel<B, R, FMT>), dim3(static_cast<uint32_t>(grid)), dim3(64 * nw),
                       0, st, reinterpret_cast<const uint4*>(packed), absmax_q, absmax2, code2,
                       offset, static_cast<int>(N), static_cast<int>(K), lbs, ls2, x, y);
  } else {
    const int64_t grid = (N + 3) / 4;
    if (grid > 0x7FFFFFFF) return NF4_EUNSUPPORTED;
    hipLaunchKernelGGL((gemv_any_kernel<B, FMT>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st,
                       packed, absmax_q, absmax2, code2, offset, N, K, lbs, ls2, x, y);
  }
  return launch_status();
}

// y = +0 for N x batch outputs (empty sums, K == 0).
nf4_status gemv_fill_zero(uint16_t* y, int64_t N, int32_t batch, hipStream_t st) {
  if (N > kMaxElems) return NF4_EUNSUPPORTED;
  const int64_t count = N * batch;
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<uint32_t>(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, st, y, count);
  return launch_status();
}

// The descriptors of the other formats share nf4_gemv_desc's layout, so the
// kernels read them as nf4_gemv_desc (the scale arrays in the absmax_q and
// absmax2 slots, as in the single-matrix entry points).
static_assert(sizeof(nf4_absmax32_gemv_desc) == sizeof(nf4_gemv_desc) &&
                  offsetof(nf4_absmax32_gemv_desc, absmax) == offsetof(nf4_gemv_desc, absmax_q) &&
                  offsetof(nf4_absmax32_gemv_desc, x) == offsetof(nf4_gemv_desc, x) &&
                  offsetof(nf4_absmax32_gemv_desc, y) == offsetof(nf4_gemv_desc, y) &&
                  offsetof(nf4_absmax32_gemv_desc, N) == offsetof(nf4_gemv_desc, N) &&
                  offsetof(nf4_absmax32_gemv_desc, row_begin) == offsetof(nf4_gemv_desc, row_begin),
              "single-level descriptor layout");
static_assert(sizeof(int4_gemv_desc) == sizeof(nf4_gemv_desc) &&
                  offsetof(int4_gemv_desc, scales) == offsetof(nf4_gemv_desc, absmax_q) &&
                  offsetof(int4_gemv_desc, zeros) == offsetof(nf4_gemv_desc, absmax2) &&
                  offsetof(int4_gemv_desc, x) == offsetof(nf4_gemv_desc, x) &&
                  offsetof(int4_gemv_desc, y) == offsetof(nf4_gemv_desc, y) &&
                  offsetof(int4_gemv_desc, N) == offsetof(nf4_gemv_desc, N) &&
                  offsetof(int4_gemv_desc, row_begin) == offsetof(nf4_gemv_desc, row_begin),
              "INT4 descriptor layout");

// Shared checks and dispatch of the grouped entry points of the single-level
// and INT4 formats (ls2 and code2 are not used by those formats).
template <int FMT>
nf4_status grouped_other(const void* descs, int32_t count, int64_t total_rows, int64_t K,
                         int32_t blocksize, int32_t batch, void* sched, size_t sched_bytes,
                         void* stream) {
  int lbs = 0;
  if (!pow2_log2(blocksize, &lbs)) return NF4_EINVAL;
  if (count < 0 || total_rows < 0 || K < 0 || (K & 1)) return NF4_EINVAL;
  if (sched != nullptr && (!aligned(sched, 256) || sched_bytes < nf4_gemv_sched_size()))
    return NF4_EINVAL;
  if (count == 0 || total_rows == 0) return NF4_OK;
  if (!descs || !aligned(descs, 8)) return NF4_EINVAL;
  if (count > kMaxDescs || total_rows >= 0x7FFFFFFF || K == 0 || K % 32 != 0 ||
      K > 8 * kSlab || lbs < 5 || batch < 1 || batch > 8)
    return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const nf4_gemv_desc* d = static_cast<const nf4_gemv_desc*>(descs);
  const nf4_gemv_desc none{};
  unsigned* sc = static_cast<unsigned*>(sched);
  const int tr = static_cast<int>(total_rows), k = static_cast<int>(K);
  switch (batch) {
    case 1: return stream_launch<1, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 2: return stream_launch<2, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 3: return stream_launch<3, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 4: return stream_launch<4, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 5: return stream_launch<5, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 6: return stream_launch<6, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    case 7: return stream_launch<7, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
    default: return stream_launch<8, FMT>(d, none, count, tr, k, lbs, 0, nullptr, sc, st);
  }
}

}  // namespace

// The scheduling counters of nf4_gemv_grouped_noalloc: the library's own
// scratch, kSchedRegions regions of kSchedStride counters (2 KiB).  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code this name is not a device address: the address of the current GPU's
// copy comes from scratch_address().
static __device__ __align__(256) unsigned scratch[kSchedRegions * kSchedStride];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<unsigned*> g_scratch_addr[kMaxDevices];  // per device; zero-initialized

// The device address of the current GPU's copy of `scratch`, looked up with
// hipGetSymbolAddress on the first call for each device (with that device
// current) and kept; nullptr if the lookup fails.  Threads racing on the first
// call store the same address.
unsigned* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  unsigned* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return nullptr;
    p = static_cast<unsigned*>(addr);
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// The checks and dispatch shared by nf4_gemv_grouped and its no-allocation
// variant.  sc: the caller's scheduling workspace (already validated) or
// NULL; use_scratch: take the library's scratch instead (looked up only once
// the arguments have passed their checks) and clear it before use.
nf4_status grouped_double(const nf4_gemv_desc* descs, int32_t count, int64_t total_rows,
                          int64_t K, int32_t blocksize, int32_t s2_blocksize,
                          const uint16_t* code2, int32_t batch, unsigned* sc, bool use_scratch,
                          void* stream) {
  int lbs = 0, ls2 = 0;
  if (!pow2_log2(blocksize, &lbs) || !pow2_log2(s2_blocksize, &ls2)) return NF4_EINVAL;
  if (count < 0 || total_rows < 0 || K < 0 || (K & 1)) return NF4_EINVAL;
  if (count == 0 || total_rows == 0) return NF4_OK;
  if (!descs || !code2 || (reinterpret_cast<uintptr_t>(descs) & 7)) return NF4_EINVAL;
  if (count > kMaxDescs || total_rows >= 0x7FFFFFFF || K == 0 || K % 32 != 0 ||
      K > 8 * kSlab || lbs < 5 || batch < 1 || batch > 8)
    return NF4_EUNSUPPORTED;
  const bool sched_clear = use_scratch;
  if (use_scratch) {
    sc = scratch_address();
    if (sc == nullptr) return NF4_EHIP;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const nf4_gemv_desc none{};
  const int tr = static_cast<int>(total_rows), k = static_cast<int>(K);
  switch (batch) {
    case 1: return stream_launch<1, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 2: return stream_launch<2, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 3: return stream_launch<3, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 4: return stream_launch<4, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 5: return stream_launch<5, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 6: return stream_launch<6, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    case 7: return stream_launch<7, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
    default: return stream_launch<8, kFmtDouble>(descs, none, count, tr, k, lbs, ls2, code2, sc, st, sched_clear);
  }
}

}  // namespace

extern "C" {

int nf4_abi_version(void) { return 1; }

const char* nf4_status_string(int status) {
  switch (status) {
    case NF4_OK: return "NF4_OK";
    case NF4_EINVAL: return "NF4_EINVAL: invalid argument";
    case NF4_EUNSUPPORTED: return "NF4_EUNSUPPORTED: size outside the supported range";
    case NF4_EHIP: return "NF4_EHIP: HIP launch error";
    default: return "unknown nf4 status";
  }
}

nf4_status nf4_dequant(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                       const uint16_t* code2, float offset, int64_t n, int32_t blocksize,
                       int32_t s2_blocksize, void* out, int32_t out_dtype, void* stream) {
  int lbs = 0, ls2 = 0;
  if (n < 0 || !pow2_log2(blocksize, &lbs) || !pow2_log2(s2_blocksize, &ls2)) return NF4_EINVAL;
  if (out_dtype != NF4_BF16 && out_dtype != NF4_FP16) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!packed || !absmax_q || !absmax2 || !code2 || !out) return NF4_EINVAL;
  if (n >= kMaxElems) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (out_dtype == NF4_BF16)
    return dequant_launch<NF4_BF16, kFmtDouble>(packed, absmax_q, absmax2, code2, offset, n, lbs,
                                                ls2, out, st);
  return dequant_launch<NF4_FP16, kFmtDouble>(packed, absmax_q, absmax2, code2, offset, n, lbs, ls2,
                                              out, st);
}

nf4_status nf4_gemv(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                    const uint16_t* code2, float offset, int64_t N, int64_t K,
                    int32_t blocksize, int32_t s2_blocksize, const uint16_t* x, int32_t batch,
                    uint16_t* y, void* stream) {
  int lbs = 0, ls2 = 0;
  if (N < 0 || K < 0 || (K & 1) || batch < 1 || batch > 8) return NF4_EINVAL;
  if (!pow2_log2(blocksize, &lbs) || !pow2_log2(s2_blocksize, &ls2)) return NF4_EINVAL;
  if (N == 0) return NF4_OK;
  if (!y) return NF4_EINVAL;
  if (K == 0) return gemv_fill_zero(y, N, batch, reinterpret_cast<hipStream_t>(stream));
  if (!packed || !absmax_q || !absmax2 || !code2 || !x) return NF4_EINVAL;
  if (N > kMaxElems / K) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (batch) {
#define NF4_GEMV_CASE(BB) \
  case BB:                \
    return gemv_launch_b<BB, kFmtDouble>(packed, absmax_q, absmax2, code2, offset, N, K, lbs, ls2, \
                                         x, y, st);
    NF4_GEMV_CASE(1)
    NF4_GEMV_CASE(2)
    NF4_GEMV_CASE(3)
    NF4_GEMV_CASE(4)
    NF4_GEMV_CASE(5)
    NF4_GEMV_CASE(6)
    NF4_GEMV_CASE(7)
    NF4_GEMV_CASE(8)
#undef NF4_GEMV_CASE
  }
  return NF4_EINVAL;
}

size_t nf4_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0 || M > (int64_t(1) << 31) / 16 ||
      N * K >= (int64_t(1) << 31) || (M + 128) * K * 2 >= (int64_t(1) << 31))
    return 0;
  return nf4gemm::plan(M, N, K, ~size_t(0)).ws_bytes;
}

nf4_status nf4_gemm(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                    const uint16_t* code2, float offset, int64_t M, int64_t N, int64_t K,
                    int32_t blocksize, int32_t s2_blocksize, const uint16_t* x, uint16_t* y,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int lbs = 0, ls2 = 0;
  if (M < 0 || N < 0 || K < 0 || (K & 1)) return NF4_EINVAL;
  if (workspace && !aligned(workspace, 256)) return NF4_EINVAL;
  if (!pow2_log2(blocksize, &lbs) || !pow2_log2(s2_blocksize, &ls2)) return NF4_EINVAL;
  if (M == 0 || N == 0) return NF4_OK;
  if (!y) return NF4_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M > (int64_t(1) << 31) / 16) return NF4_EUNSUPPORTED;
  if (K == 0) {
    if (N > kMaxElems / M) return NF4_EUNSUPPORTED;
    return gemv_fill_zero(y, M * N, 1, st);
  }
  if (!packed || !absmax_q || !absmax2 || !code2 || !x) return NF4_EINVAL;
  if (N > kMaxElems / K) return NF4_EUNSUPPORTED;
  const bool fast = K % 64 == 0 && lbs >= 6 && aligned(packed, 16) && aligned(x, 16) &&
                    N * K < (int64_t(1) << 31) && (M + 128) * K * 2 < (int64_t(1) << 31);
  if (fast)
    return nf4gemm::launch(packed, absmax_q, absmax2, code2, offset, M, N, K, lbs, ls2, x, y,
                           workspace, workspace_bytes, st);
  // anything else: the GEMV over batch chunks of up to 8 rows
  for (int64_t m0 = 0; m0 < M; m0 += 8) {
    const int64_t b = M - m0 < 8 ? M - m0 : 8;
    const uint16_t* xc = x + m0 * K;
    uint16_t* yc = y + m0 * N;
    nf4_status r = NF4_OK;
    switch (b) {
#define NF4_GEMM_CHUNK(BB)                                                                        \
  case BB:                                                                                        \
    r = gemv_launch_b<BB, kFmtDouble>(packed, absmax_q, absmax2, code2, offset, N, K, lbs, ls2, \
                                      xc, yc, st);                                                \
    break;
      NF4_GEMM_CHUNK(1)
      NF4_GEMM_CHUNK(2)
      NF4_GEMM_CHUNK(3)
      NF4_GEMM_CHUNK(4)
      NF4_GEMM_CHUNK(5)
      NF4_GEMM_CHUNK(6)
      NF4_GEMM_CHUNK(7)
      NF4_GEMM_CHUNK(8)
#undef NF4_GEMM_CHUNK
    }
    if (r != NF4_OK) return r;
  }
  return NF4_OK;
}

nf4_status nf4_dequant_absmax32(const uint8_t* packed, const float* absmax, int64_t n,
                                int32_t blocksize, void* out, int32_t out_dtype, void* stream) {
  int lbs = 0;
  if (n < 0 || !pow2_log2(blocksize, &lbs)) return NF4_EINVAL;
  if (out_dtype != NF4_BF16 && out_dtype != NF4_FP16) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!packed || !absmax || !out || !aligned(absmax, 4)) return NF4_EINVAL;
  if (n >= kMaxElems) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* am = reinterpret_cast<const uint8_t*>(absmax);
  if (out_dtype == NF4_BF16)
    return dequant_launch<NF4_BF16, kFmtAbsmax32>(packed, am, nullptr, nullptr, 0.0f, n, lbs, 0,
                                                  out, st);
  return dequant_launch<NF4_FP16, kFmtAbsmax32>(packed, am, nullptr, nullptr, 0.0f, n, lbs, 0, out,
                                                st);
}

nf4_status nf4_gemv_absmax32(const uint8_t* packed, const float* absmax, int64_t N, int64_t K,
                             int32_t blocksize, const uint16_t* x, int32_t batch, uint16_t* y,
                             void* stream) {
  int lbs = 0;
  if (N < 0 || K < 0 || (K & 1) || batch < 1 || batch > 8) return NF4_EINVAL;
  if (!pow2_log2(blocksize, &lbs)) return NF4_EINVAL;
  if (N == 0) return NF4_OK;
  if (!y) return NF4_EINVAL;
  if (K == 0) return gemv_fill_zero(y, N, batch, reinterpret_cast<hipStream_t>(stream));
  if (!packed || !absmax || !x || !aligned(absmax, 4)) return NF4_EINVAL;
  if (N > kMaxElems / K) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* am = reinterpret_cast<const uint8_t*>(absmax);
  switch (batch) {
#define NF4_GEMV_SL_CASE(BB)                                                                  \
  case BB:                                                                                    \
    return gemv_launch_b<BB, kFmtAbsmax32>(packed, am, nullptr, nullptr, 0.0f, N, K, lbs, 0, x, \
                                           y, st);
    NF4_GEMV_SL_CASE(1)
    NF4_GEMV_SL_CASE(2)
    NF4_GEMV_SL_CASE(3)
    NF4_GEMV_SL_CASE(4)
    NF4_GEMV_SL_CASE(5)
    NF4_GEMV_SL_CASE(6)
    NF4_GEMV_SL_CASE(7)
    NF4_GEMV_SL_CASE(8)
#undef NF4_GEMV_SL_CASE
  }
  return NF4_EINVAL;
}

nf4_status int4_dequant(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                        int64_t n, int32_t group_size, void* out, int32_t out_dtype,
                        void* stream) {
  int lg = 0;
  if (n < 0 || !pow2_log2(group_size, &lg) || lg < 1) return NF4_EINVAL;
  if (out_dtype != NF4_BF16 && out_dtype != NF4_FP16) return NF4_EINVAL;
  if (n == 0) return NF4_OK;
  if (!packed || !scales || !zeros || !out) return NF4_EINVAL;
  if (n >= kMaxElems) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
  if (out_dtype == NF4_BF16)
    return dequant_launch<NF4_BF16, kFmtInt4>(packed, sc, zeros, nullptr, 0.0f, n, lg, 0, out, st);
  return dequant_launch<NF4_FP16, kFmtInt4>(packed, sc, zeros, nullptr, 0.0f, n, lg, 0, out, st);
}

nf4_status int4_gemv(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, int32_t group_size, const uint16_t* x, int32_t batch,
                     uint16_t* y, void* stream) {
  int lg = 0;
  if (N < 0 || K < 0 || (K & 1) || batch < 1 || batch > 8) return NF4_EINVAL;
  if (!pow2_log2(group_size, &lg) || lg < 1) return NF4_EINVAL;
  if (N == 0) return NF4_OK;
  if (!y) return NF4_EINVAL;
  if (K == 0) return gemv_fill_zero(y, N, batch, reinterpret_cast<hipStream_t>(stream));
  if (!packed || !scales || !zeros || !x) return NF4_EINVAL;
  if (N > kMaxElems / K) return NF4_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
  switch (batch) {
#define INT4_GEMV_CASE(BB) \
  case BB:                 \
    return gemv_launch_b<BB, kFmtInt4>(packed, sc, zeros, nullptr, 0.0f, N, K, lg, 0, x, y, st);
    INT4_GEMV_CASE(1)
    INT4_GEMV_CASE(2)
    INT4_GEMV_CASE(3)
    INT4_GEMV_CASE(4)
    INT4_GEMV_CASE(5)
    INT4_GEMV_CASE(6)
    INT4_GEMV_CASE(7)
    INT4_GEMV_CASE(8)
#undef INT4_GEMV_CASE
  }
  return NF4_EINVAL;
}

size_t nf4_gemv_sched_size(void) {
  return sizeof(unsigned) * kSchedRegions * kSchedStride;
}

nf4_status nf4_gemv_grouped_absmax32(const nf4_absmax32_gemv_desc* descs, int32_t count,
                                     int64_t total_rows, int64_t K, int32_t blocksize,
                                     int32_t batch, void* sched, size_t sched_bytes,
                                     void* stream) {
  return grouped_other<kFmtAbsmax32>(descs, count, total_rows, K, blocksize, batch, sched,
                                     sched_bytes, stream);
}

nf4_status int4_gemv_grouped(const int4_gemv_desc* descs, int32_t count, int64_t total_rows,
                             int64_t K, int32_t group_size, int32_t batch, void* sched,
                             size_t sched_bytes, void* stream) {
  return grouped_other<kFmtInt4>(descs, count, total_rows, K, group_size, batch, sched,
                                 sched_bytes, stream);
}

nf4_status nf4_gemv_grouped(const nf4_gemv_desc* descs, int32_t count, int64_t total_rows,
                            int64_t K, int32_t blocksize, int32_t s2_blocksize,
                            const uint16_t* code2, int32_t batch, void* sched,
                            size_t sched_bytes, void* stream) {
  if (sched != nullptr && (!aligned(sched, 256) || sched_bytes < nf4_gemv_sched_size()))
    return NF4_EINVAL;
  return grouped_double(descs, count, total_rows, K, blocksize, s2_blocksize, code2, batch,
                        static_cast<unsigned*>(sched), false, stream);
}

nf4_status nf4_gemv_grouped_noalloc(const nf4_gemv_desc* descs, int32_t count,
                                    int64_t total_rows, int64_t K, int32_t blocksize,
                                    int32_t s2_blocksize, const uint16_t* code2, int32_t batch,
                                    void* stream) {
  static_assert(sizeof(scratch) == sizeof(unsigned) * kSchedRegions * kSchedStride,
                "the scratch holds exactly one scheduling workspace");
  // the workspace a launch needs is the same fixed size for every launch, so
  // no launch size can exceed the scratch; the grouped limits still apply
  if (nf4_gemv_sched_size() > sizeof(scratch)) return NF4_EUNSUPPORTED;
  return grouped_double(descs, count, total_rows, K, blocksize, s2_blocksize, code2, batch,
                        nullptr, true, stream);
}

nf4_status nf4_gemv_desc_check(const void* descs, int32_t count, int64_t total_rows, int64_t K,
                               int32_t format, int32_t* first_bad) {
  if (first_bad) *first_bad = -1;
  if (count < 0 || total_rows < 0 || K < 0 || format < 0 || format > 2) return NF4_EINVAL;
  if (count == 0) return total_rows == 0 ? NF4_OK : NF4_EINVAL;
  if (descs == nullptr) return NF4_EINVAL;
  const nf4_gemv_desc* d = static_cast<const nf4_gemv_desc*>(descs);
  int64_t row = 0;
  for (int32_t i = 0; i < count; ++i) {
    const nf4_gemv_desc& e = d[i];
    const uintptr_t sa = reinterpret_cast<uintptr_t>(e.absmax_q);
    const uintptr_t za = reinterpret_cast<uintptr_t>(e.absmax2);
    const bool scales_ok = format == kFmtAbsmax32 ? (sa & 3) == 0
                           : format == kFmtInt4   ? ((sa | za) & 1) == 0
                                                  : (za & 1) == 0;
    const bool ok = e.packed && e.absmax_q && (format == kFmtAbsmax32 || e.absmax2) && e.x &&
                    e.y && aligned(e.packed, 16) && aligned(e.x, 16) && scales_ok && e.N >= 0 &&
                    e.N <= 0x7FFFFFFF && e.N * K < (int64_t(1) << 31) && e.row_begin == row;
    if (!ok) {
      if (first_bad) *first_bad = i;
      return NF4_EINVAL;
    }
    row += e.N;
  }
  if (row != total_rows) {
    if (first_bad) *first_bad = count;
    return NF4_EINVAL;
  }
  return NF4_OK;
}

}  // extern "C"
