// nf4_gemm.hip -- the NF4 W4A16 product on the matrix cores (batch rows past
// 8, prefill) behind nf4_gemm ([quanttax] "Kernel 实现" and its conclusions on
// prefill; [handbook] batch sensitivity).  Same decode table, block indexing
// and scale reconstruction as the GEMV in nf4_kernels.hip ([report] §1.3).
//
// Pages (by title): [report] "NF4 双重量化反量化 CUDA Kernel 实现报告";
// [quanttax] "RTX 4060 上的 LLM 量化实测"; [handbook] "量化与 GEMV".

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4.h"
#include "nf4_device.h"
#include "nf4_gemm.h"

namespace {

using namespace nf4dev;

// ---------------------------------------------------------------------------
// Batched NF4 W4A16 GEMM on the matrix cores (batch 9 and up, prefill):
// y[m][n] = sum_k value(n K + k) * x[m][k].
//
// v_mfma_f32_16x16x32_bf16 with the activations as A (16 batch rows x 32 k)
// and the decoded weights as B (32 k x 16 columns n).  Lane layout (checked on
// gfx950): A lane i + 16 g holds A[i][8 g .. 8 g + 7], B lane j + 16 g holds
// B[8 g .. 8 g + 7][j], D lane j + 16 g holds D[4 g .. 4 g + 3][j] -- so a
// lane's B column is also its D column.
//
// Tiling.  A workgroup of eight waves owns 64 columns and 16 MT batch rows,
// over one of SK equal ranges of the K blocks (64 columns each), taken two
// blocks at a time: waves 0-3 compute the even block of each pair and waves
// 4-7 the odd one, wave w on columns 16 (w % 4) .. + 15, so every SIMD runs
// two waves.  The activation tiles of a pair (2 x 16 MT rows x 128 bytes) are
// loaded once per workgroup with whole-cache-line loads (eight lanes per row),
// kept in registers for one pair and then written to one of two LDS buffers
// (rows padded to 144 bytes, so the MFMA operand reads of 16 rows hit distinct
// banks).  Each wave loads and decodes only its own columns: per block lane
// (j, g) takes the 8 packed bytes of k [16 g, 16 g + 16) of its row and
// decodes them through the pair table into bf16 hi pairs and lo pairs (hi +
// lo within 2^-16 of the NF4 value).  Two k-steps of 32 times (hi, lo) are
// four MFMAs per 16 x 16 tile, summed unscaled; the block's absmax_real of the
// column then multiplies that sum into the lane's fp32 accumulator (scale
// after accumulate, as in the GEMV).  One barrier per pair.  At the end the
// odd-block waves hand their sums to the even-block waves through LDS (a
// fixed-order sum).
//
// Split K (SK > 1, when the column tiles alone would leave compute units
// idle): each workgroup writes its fp32 partial tile to plane `split` of the
// workspace, and a second kernel sums the planes in split order into bf16 y.
// (A handoff inside the kernel would need device-scope release/acquire
// fences, which write back and invalidate the L2 of this multi-XCD part: far
// slower than the second launch.)
// Requirements (checked on the host): K % 64 == 0, blocksize >= 64, packed
// 8-byte aligned, x 16-byte aligned, N K < 2^31, (M + 128) K 2 < 2^31.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kGemmThreads = 512;
constexpr int kGemmXRow = 144;  // LDS bytes per activation row (128 + 16 of padding)

// Activation chunks of 16 bytes per pair: 2 blocks x 16 MT rows x 8; each of
// the 512 threads loads MT / 2 of them (at MT = 1 half the threads load one).
template <int MT>
constexpr int gemm_xloads() { return MT >= 2 ? MT / 2 : 1; }

template <int MT, int NT>
struct GemmStage {
  u32x4 xg[gemm_xloads<MT>()];  // activation chunks this thread loads
  uint2 w[NT];                  // 8 packed bytes per column of the lane, its block of the pair
  uint32_t q[NT];               // absmax_q of that block
  uint32_t a2[NT];              // absmax2 of its group
};

template <int NT>
struct GemmLane {
  __amdgpu_buffer_rsrc_t rp, rq, ra2, rx;
  uint32_t wrow[NT];     // byte offset of the lane's weight rows (kFar past N)
  uint32_t blk_row[NT];  // flat index of each row's first element
  uint32_t g;        // k-group of the lane (0..3)
  uint32_t par;      // block of the pair the wave computes (0 or 1)
  uint32_t xg_off[4];  // byte offsets of this thread's activation chunks (pair 0)
  bool xg_live;        // whether the thread loads activation chunks at all
  int log2bs, log2s2;
};

template <int MT, int NT>
__device__ __forceinline__ void gemm_load(GemmStage<MT, NT>& st, int kp, int kb1,
                                          const GemmLane<NT>& L) {
  const uint32_t kb = 2u * static_cast<uint32_t>(kp) + L.par;
  const uint32_t far = static_cast<int>(kb) < kb1 ? 0u : kFar;
  const uint32_t kcol = kb * 64u;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.w[nt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                             L.rp, L.wrow[nt] + kcol / 2u + 8u * L.g, far,
                                             kStreamLoad));
    const uint32_t blk = (L.blk_row[nt] + kcol) >> L.log2bs;
    st.q[nt] = __builtin_amdgcn_raw_buffer_load_b8(L.rq, blk, far, 0);
    st.a2[nt] = __builtin_amdgcn_raw_buffer_load_b16(L.ra2, (blk >> L.log2s2) * 2u, far, 0);
  }
  // the pair's activations (a block past kb1 reads as zeros)
  const uint32_t pfar = 2 * kp < kb1 && L.xg_live ? 0u : kFar;
#pragma unroll
  for (int i = 0; i < gemm_xloads<MT>(); ++i)
    st.xg[i] = __builtin_amdgcn_raw_buffer_load_b128(
        L.rx, L.xg_off[i] + static_cast<uint32_t>(kp) * 256u, pfar, 0);
}

// This thread's activation chunks of a stage into an LDS buffer; chunk c of
// the pair is block c / (128 MT), row (c / 8) % (16 MT), bytes (c % 8) 16.
template <int MT, int NT>
__device__ __forceinline__ void gemm_stash(const GemmStage<MT, NT>& st, char* buf, int tid) {
  constexpr int XTILE = 16 * MT * kGemmXRow;
  if (MT >= 2 || tid < 256) {
#pragma unroll
    for (int i = 0; i < gemm_xloads<MT>(); ++i) {
      const int c = tid + kGemmThreads * i;
      const int b = c / (128 * MT), r = (c >> 3) % (16 * MT);
      *reinterpret_cast<u32x4*>(buf + b * XTILE + r * kGemmXRow + (c & 7) * 16) = st.xg[i];
    }
  }
}

template <int MT, int NT>
__device__ __forceinline__ void gemm_block(const GemmStage<MT, NT>& st, const char* tab,
                                           const char* xbuf, uint32_t copy_off, int lane,
                                           const float* s_code2, float offset,
                                           f32x4 (&acc)[MT][NT]) {
  const int i = lane & 15, g = lane >> 4;
  // B operands: byte 4 t + e of the lane's 8 bytes holds k 16 g + 8 t + 2 e, + 1;
  // one 8-byte table read gives its hi and lo pairs (conflict-free: lanes l
  // and l + 16 read the two halves of one bank pair)
  bf16x8 bhv[NT][2], blv[NT][2];
  float a[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t word = t == 0 ? st.w[nt].x : st.w[nt].y;
      uint2 e2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t addr = __builtin_amdgcn_perm(copy_off, word, 0x0C0C0004u | (uint32_t(e) << 8));
        e2[e] = *reinterpret_cast<const uint2*>(tab + addr);
      }
      bhv[nt][t] = __builtin_bit_cast(bf16x8, (u32x4){e2[0].x, e2[1].x, e2[2].x, e2[3].x});
      blv[nt][t] = __builtin_bit_cast(bf16x8, (u32x4){e2[0].y, e2[1].y, e2[2].y, e2[3].y});
    }
    const float prod = s_code2[st.q[nt] & 0xFFu] * f16_to_f32(static_cast<uint16_t>(st.a2[nt]));
    a[nt] = prod + offset;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // A operands: row 16 mt + i, k 16 g + 8 t .. + 7
    const char* row = xbuf + (16 * mt + i) * kGemmXRow + 32 * g;
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row));
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, bhv[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, blv[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, bhv[nt][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, blv[nt][1], c, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][nt][r] += a[nt] * c[r];
    }
  }
}

template <int MT, int NT>
__global__ __launch_bounds__(kGemmThreads) void gemm_mfma_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ absmax_q,
    const uint16_t* __restrict__ absmax2, const uint16_t* __restrict__ code2, float offset, int M,
    int N, int K, int log2bs, int log2s2, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, float* __restrict__ part, int SK) {
  constexpr int BM = 16 * MT;
  constexpr int XPAIR = 2 * BM * kGemmXRow;  // LDS bytes of one pair's activations
  static_assert(4 * MT * NT * 64 * sizeof(f32x4) <= 256 * kPairCopies * sizeof(uint2),
                "the odd-block sums fit in the decode table's LDS");
  __shared__ uint2 s_pairs[256 * kPairCopies];  // 64 KiB decode table
  __shared__ float s_code2[256];
  __shared__ __attribute__((aligned(16))) char s_x[2 * XPAIR];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  // the lane's columns: n0 + 16 nt, nt < NT
  const int n0 = blockIdx.x * (64 * NT) + (wave & 3) * (16 * NT) + j;
  const int m0 = blockIdx.y * BM;
  const int split = blockIdx.z;

  GemmLane<NT> L;
  const uint64_t nk = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  const uint64_t nb = ((nk - 1) >> log2bs) + 1;
  const uint64_t ng = ((nb - 1) >> log2s2) + 1;
  L.rp = rsrc(packed, static_cast<uint32_t>(nk >> 1));
  L.rq = rsrc(absmax_q, static_cast<uint32_t>(nb));
  L.ra2 = rsrc(absmax2, static_cast<uint32_t>(ng * 2));
  L.rx = rsrc(x, static_cast<uint32_t>(static_cast<uint64_t>(M) * K * 2));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt;
    L.wrow[nt] = n < N ? static_cast<uint32_t>(n) * static_cast<uint32_t>(K >> 1) : kFar;
    L.blk_row[nt] = static_cast<uint32_t>(n < N ? n : 0) * static_cast<uint32_t>(K);
  }
  L.g = static_cast<uint32_t>(g);
  L.par = static_cast<uint32_t>(wave >> 2);
  L.xg_live = MT >= 2 || tid < 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kGemmThreads * i;
    const int b = c / (128 * MT), r = (c >> 3) % (16 * MT);
    L.xg_off[i] = static_cast<uint32_t>(m0 + r) * static_cast<uint32_t>(K) * 2u +
                  static_cast<uint32_t>(b) * 128u + static_cast<uint32_t>(c & 7) * 16u;
  }
  L.log2bs = log2bs;
  L.log2s2 = log2s2;

  // this workgroup's range of K blocks, taken in pairs from kb0 (even)
  const int nkb = K >> 6;
  const int kb0 = (split * nkb / SK) & ~1, kb1 = split + 1 == SK ? nkb : ((split + 1) * nkb / SK) & ~1;
  const int kp0 = kb0 >> 1, kp1 = (kb1 + 1) >> 1;
  GemmStage<MT, NT> st[3];
  gemm_load<MT, NT>(st[0], kp0, kb1, L);
  gemm_load<MT, NT>(st[1], kp0 + 1, kb1, L);

  if (tid < 256) s_code2[tid] = f16_to_f32(code2[tid]);
  build_pair_table(s_pairs, tid, blockDim.x);
  const uint32_t copy_off = static_cast<uint32_t>(lane % kPairCopies) * 8u;
  gemm_stash<MT, NT>(st[0], s_x, tid);
  __syncthreads();
  const char* tab = reinterpret_cast<const char*>(s_pairs);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // pair kp: its activations are in LDS buffer (kp - kp0) & 1, the wave's
  // weights in st[(kp - kp0) % 3]; the loads of pair kp + 2 go out before it
  // is computed and pair kp + 1's activations are stashed after it
  for (int kp = kp0; kp < kp1; kp += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int p = kp + u;
      if (p < kp1) {
        gemm_load<MT, NT>(st[(u + 2) % 3], p + 2, kb1, L);
        if (2 * p + static_cast<int>(L.par) < kb1) {
          const char* xbuf = s_x + ((p - kp0) & 1) * XPAIR + L.par * (XPAIR / 2);
          gemm_block<MT, NT>(st[u], tab, xbuf, copy_off, lane, s_code2, offset, acc);
        }
        gemm_stash<MT, NT>(st[(u + 1) % 3], s_x + ((p + 1 - kp0) & 1) * XPAIR, tid);
        __syncthreads();
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // the odd-block waves' sums go to the even-block waves through the table's
  // LDS (every wave is past its last table read: the loop ends on a barrier)
  f32x4* s_red = reinterpret_cast<f32x4*>(s_pairs);  // [4 waves][MT][NT][64]
  if (wave >= 4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        s_red[(((wave - 4) * MT + mt) * NT + nt) * 64 + lane] = acc[mt][nt];
  }
  __syncthreads();
  if (wave >= 4) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const f32x4 o = s_red[((wave * MT + mt) * NT + nt) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][nt][r] += o[r];
    }
  // SK == 1: the bf16 tile; else the partial tile into plane `split` of the
  // workspace (summed by gemm_reduce_kernel)
  float* dst = SK > 1 ? part + static_cast<int64_t>(split) * M * N : nullptr;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mt + 4 * g + r;
        if (m >= M) continue;
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if (SK > 1)
          dst[o] = acc[mt][nt][r];
        else
          y[o] = to_half_bits<NF4_BF16>(acc[mt][nt][r]);
      }
  }
}

// y = bf16 of the sum of the SK partial planes, in split order (the same
// bits whichever workgroup finished first).  Four outputs per thread when N
// is a multiple of 4.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part,
                                                          uint16_t* __restrict__ y, int64_t count,
                                                          int SK, int vec4) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  if (vec4) {
    const int64_t n4 = count >> 2;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
         i += stride) {
      float4 v = reinterpret_cast<const float4*>(part)[i];
      for (int s = 1; s < SK; ++s) {
        const float4 p = reinterpret_cast<const float4*>(part + s * count)[i];
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
      }
      const uint2 o = make_uint2(pack_pair<NF4_BF16>(v.x, v.y), pack_pair<NF4_BF16>(v.z, v.w));
      reinterpret_cast<uint2*>(y)[i] = o;
    }
  } else {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += stride) {
      float v = part[i];
      for (int s = 1; s < SK; ++s) v += part[s * count + i];
      y[i] = to_half_bits<NF4_BF16>(v);
    }
  }
}

}  // namespace

namespace nf4gemm {

using namespace nf4dev;

// Launch shape of the MFMA GEMM: MT row tiles of 16 per workgroup (1, 2, 4
// or 8), 64 columns per workgroup, SK splits of the K blocks.  SK is chosen
// to minimise (rounds of workgroups over the compute units) x (blocks per
// workgroup + a fixed cost of about 8 blocks per workgroup: table build and
// first loads), among the splits whose partial sums fit in `ws_avail` bytes;
// a split must save an eighth of that time to pay for its partial sums.
static size_t gemm_ws_bytes(int64_t M, int64_t N, int SK) {
  if (SK <= 1) return 0;
  return static_cast<size_t>(SK) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
}

Plan plan(int64_t M, int64_t N, int64_t K, size_t ws_avail) {
  Plan p{};
  const int64_t tm = (M + 15) / 16;
  p.MT = tm >= 5 ? 8 : tm >= 3 ? 4 : static_cast<int>(tm);
  p.NT = 1;  // 32 columns per wave (NT = 2) measured slower: fewer workgroups, same stalls
  p.gx = (N + 64 * p.NT - 1) / (64 * p.NT);
  p.gy = (M + 16 * p.MT - 1) / (16 * p.MT);
  const int64_t tiles = p.gx * p.gy;
  // one workgroup per CU (two at MT = 1: LDS)
  const int64_t slots = static_cast<int64_t>(device_cus()) * (p.MT == 1 ? 2 : 1);
  const int64_t nkb = K / 64;
  p.SK = 1;
  constexpr int64_t kFixed = 8;  // per-workgroup cost in blocks
  int64_t best = ((tiles + slots - 1) / slots) * (nkb + kFixed);
  for (int sk = 2; sk <= 8; ++sk) {
    if (nkb < 4 * sk) break;
    const size_t ws = gemm_ws_bytes(M, N, sk);
    if (ws > ws_avail) break;
    const int64_t cost = ((tiles * sk + slots - 1) / slots) * ((nkb + sk - 1) / sk + kFixed);
    if (cost * 8 < best * 7) {
      best = cost;
      p.SK = sk;
    }
  }
  p.ws_bytes = gemm_ws_bytes(M, N, p.SK);
  return p;
}

nf4_status launch(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                  const uint16_t* code2, float offset, int64_t M, int64_t N, int64_t K, int lbs,
                  int ls2, const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes,
                  hipStream_t st) {
  const Plan p = plan(M, N, K, ws ? ws_bytes : 0);
  if (p.gy > 65535 || p.gx > 0x7FFFFFFF) return NF4_EUNSUPPORTED;
  const dim3 grid(static_cast<uint32_t>(p.gx), static_cast<uint32_t>(p.gy),
                  static_cast<uint32_t>(p.SK));
  const dim3 block(kGemmThreads);
  float* part = p.SK > 1 ? static_cast<float*>(ws) : nullptr;
  const int m = static_cast<int>(M), nn = static_cast<int>(N), k = static_cast<int>(K);
  switch (p.MT * 4 + p.NT) {
#define NF4_GEMM_MT(T, U)                                                                       \
  case T * 4 + U:                                                                               \
    hipLaunchKernelGGL((gemm_mfma_kernel<T, U>), grid, block, 0, st, packed, absmax_q, absmax2, \
                       code2, offset, m, nn, k, lbs, ls2, x, y, part, p.SK);                     \
    break;
    NF4_GEMM_MT(1, 1)
    NF4_GEMM_MT(2, 1)
    NF4_GEMM_MT(4, 1)
    NF4_GEMM_MT(8, 1)
#undef NF4_GEMM_MT
    default: return NF4_EINVAL;
  }
  if (p.SK > 1) {
    const int64_t count = M * N;
    const int vec4 = N % 4 == 0 && aligned(y, 8);
    const int64_t items = vec4 ? count / 4 : count;
    const int64_t blocks = (items + 255) / 256;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(static_cast<uint32_t>(blocks < 8192 ? blocks : 8192)),
                       dim3(256), 0, st, part, y, count, p.SK, vec4);
  }
  return launch_status();
}

}  // namespace nf4gemm
