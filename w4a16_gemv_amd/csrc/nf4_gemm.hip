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
// over one of SK ranges of the K blocks (64 columns each), taken 2 R blocks
// (a group) at a time: waves 0-3 compute the first R blocks of each group and
// waves 4-7 the last R, wave w on columns 16 (w % 4) .. + 15, so every SIMD
// runs two waves.  The activation tiles of a group (2 R x 16 MT rows x 128
// bytes) are loaded once per workgroup with whole-cache-line loads (eight
// lanes per row), kept in registers for one group and then written to one of
// two LDS buffers (rows padded to 144 bytes, so the MFMA operand reads of 16
// rows hit distinct banks); all waves read their A operands from there.  One
// barrier per group.
//
// Each wave loads and decodes only its own columns.  R = 1 (16 MT >= 64 rows):
// lane (j, g) loads the 8 packed bytes of k [16 g, 16 g + 16) of its row and
// block.  R = 4 (fewer rows, where the per-block latency and the weight
// stream dominate): lane (j, g) loads the whole 32 bytes of block g of its
// row's four (the wave reads 16 rows x 128 bytes, whole lines), and a 4 x 4
// transpose of 8-byte units across the four 16-lane rows (two
// v_permlane32_swap and two v_permlane16_swap per dword pair) hands lane
// (j, g) bytes [8 g, 8 g + 8) of each block.  The bytes are decoded through
// the pair table into bf16 hi pairs and lo pairs (hi + lo within 2^-16 of the
// NF4 value).  Two k-steps of 32 times (hi, lo) are four MFMAs per 16 x 16
// tile, summed unscaled; the block's absmax_real of the column then multiplies
// that sum into the lane's fp32 accumulator (scale after accumulate, as in the
// GEMV).  At the end the second-half waves hand their sums to the first-half
// waves through LDS (a fixed-order sum).
//
// Split K (SK > 1, when the column tiles alone would leave compute units
// idle): each workgroup writes its fp32 partial tile to plane `split` of the
// workspace, and a second kernel sums the planes in split order into bf16 y.
// (A handoff inside the kernel would need device-scope release/acquire
// fences, which write back and invalidate the L2 of this multi-XCD part: far
// slower than the second launch.)
// Requirements (checked on the host): K % 64 == 0, blocksize >= 64, packed
// 16-byte aligned, x 16-byte aligned, N K < 2^31, (M + 128) K 2 < 2^31.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kGemmThreads = 512;
constexpr int kGemmXRow = 144;  // LDS bytes per activation row (128 + 16 of padding)

// Blocks per wave and group: 4 below 64 rows, 1 from 64 rows on.
template <int MT>
constexpr int gemm_r() { return MT <= 2 ? 4 : 1; }

// Activation chunks of 16 bytes per group: 2 R blocks x 16 MT rows x 8; each
// of the 512 threads loads R MT / 2 of them (at R MT = 1 half the threads load
// one).
// Register stages of loads in flight (S - 1 groups ahead of the one computed).
// Deeper pipelines measured slower (M = 16, 11008 x 4096: 21.9 / 24.6 / 32.5
// us at 3 / 6 / 10 stages).
template <int MT>
constexpr int gemm_stages() { return 3; }

template <int MT>
constexpr int gemm_xloads() { return gemm_r<MT>() * MT >= 2 ? gemm_r<MT>() * MT / 2 : 1; }

template <int MT>
struct GemmStage {
  u32x4 xg[gemm_xloads<MT>()];  // activation chunks this thread loads
  uint32_t w[gemm_r<MT>()][2];  // 8 packed bytes of each of the wave's blocks (lane layout)
  uint32_t q[gemm_r<MT>()];     // absmax_q of each block
  uint32_t a2[gemm_r<MT>()];    // absmax2 of its group
};

struct GemmLane {
  __amdgpu_buffer_rsrc_t rp, rq, ra2, rx;
  uint32_t wrow;        // byte offset of the lane's weight row (kFar past N)
  uint32_t blk_row;     // flat index of that row's first element
  uint32_t g;           // k-group of the lane (0..3)
  uint32_t half;        // which R blocks of each group the wave computes (0 or 1)
  uint32_t xg_off[16];  // byte offsets of this thread's activation chunks (group 0)
  bool xg_live;         // whether the thread loads activation chunks at all
  int log2bs, log2s2;
};

// The four blocks of a lane's row as loaded (see gemm_load): lane row g
// holds the 8-byte units 2 (g & 1) and 2 (g & 1) + 1 of block g >> 1 in
// u[0], u[1] and of block 2 + (g >> 1) in u[2], u[3].  One v_permlane32_swap
// per dword of the slot pairs (0, 1) and (2, 3) exchanges the high bit of the
// lane row with the low bit of the slot; afterwards u[b] of lane row g holds
// unit unit_of_row(g) of block b.
__device__ __forceinline__ void gather_units(uint32_t (&u)[4][2]) {
#pragma unroll
  for (int p = 0; p < 4; p += 2)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const auto s = __builtin_amdgcn_permlane32_swap(u[p][d], u[p + 1][d], false, false);
      u[p][d] = s[0];
      u[p + 1][d] = s[1];
    }
}

// The unit (k 16 u .. 16 u + 15 of a block) that lane row g holds after
// gather_units: the two bits of g swapped.
__device__ __forceinline__ int unit_of_row(int g) { return ((g & 1) << 1) | (g >> 1); }

template <int MT>
__device__ __forceinline__ void gemm_load(GemmStage<MT>& st, int grp, int kb1, const GemmLane& L) {
  constexpr int R = gemm_r<MT>();
  const uint32_t kbw = static_cast<uint32_t>(grp) * (2u * R) + L.half * R;  // the wave's first block
  if constexpr (R == 4) {
    // the 128 bytes of blocks kbw .. kbw + 3 of the lane's row: lane row g
    // loads bytes [16 g, +16) (block g >> 1) and [64 + 16 g, +16) (block 2 +
    // (g >> 1)), so each load instruction reads 64 contiguous bytes of each
    // of its 16 rows (two loads at 32 g and 32 g + 16 would each cover half
    // of every line in 16-byte pieces, a slower pattern); gather_units then
    // regroups the units.  A block past kb1 is pushed out of range in the
    // lane's VGPR offset: a lane-dependent scalar offset would make the
    // compiler loop over its distinct values around every load
    const uint32_t b0 = kbw + (L.g >> 1), b1 = b0 + 2u;
    const uint32_t base = L.wrow + kbw * 32u + 16u * L.g;
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(
        L.rp, base + (static_cast<int>(b0) < kb1 ? 0u : kFar), 0u, kStreamLoad);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(
        L.rp, base + 64u + (static_cast<int>(b1) < kb1 ? 0u : kFar), 0u, kStreamLoad);
    st.w[0][0] = lo[0]; st.w[0][1] = lo[1]; st.w[1][0] = lo[2]; st.w[1][1] = lo[3];
    st.w[2][0] = hi[0]; st.w[2][1] = hi[1]; st.w[3][0] = hi[2]; st.w[3][1] = hi[3];
  } else {
    const uint32_t far = static_cast<int>(kbw) < kb1 ? 0u : kFar;
    const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  L.rp, L.wrow + kbw * 32u + 8u * L.g, far,
                                                  kStreamLoad));
    st.w[0][0] = w.x;
    st.w[0][1] = w.y;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t kb = kbw + r;
    const uint32_t far = static_cast<int>(kb) < kb1 ? 0u : kFar;
    const uint32_t blk = (L.blk_row + kb * 64u) >> L.log2bs;
    st.q[r] = __builtin_amdgcn_raw_buffer_load_b8(L.rq, blk, far, 0);
    st.a2[r] = __builtin_amdgcn_raw_buffer_load_b16(L.ra2, (blk >> L.log2s2) * 2u, far, 0);
  }
  // the group's activations (blocks past kb1 read as zeros or are never used)
  const uint32_t gfar = static_cast<int>(grp * 2 * R) < kb1 ? 0u : kFar;  // uniform
#pragma unroll
  for (int i = 0; i < gemm_xloads<MT>(); ++i)
    st.xg[i] = __builtin_amdgcn_raw_buffer_load_b128(
        L.rx, L.xg_off[i] + static_cast<uint32_t>(grp) * (256u * R), gfar, 0);
}

// This thread's activation chunks of a stage into an LDS buffer; chunk c of
// the group is block c / (128 MT), row (c / 8) % (16 MT), bytes (c % 8) 16.
template <int MT>
__device__ __forceinline__ void gemm_stash(const GemmStage<MT>& st, char* buf, int tid) {
  constexpr int XTILE = 16 * MT * kGemmXRow;
  if (gemm_r<MT>() * MT >= 2 || tid < 256) {
#pragma unroll
    for (int i = 0; i < gemm_xloads<MT>(); ++i) {
      const int c = tid + kGemmThreads * i;
      const int b = c / (128 * MT), r = (c >> 3) % (16 * MT);
      *reinterpret_cast<u32x4*>(buf + b * XTILE + r * kGemmXRow + (c & 7) * 16) = st.xg[i];
    }
  }
}

// One block: w = the lane's 8 bytes in MFMA layout (unit `unit` of the
// block: k 16 unit .. 16 unit + 15), xbuf = the block's activation tile.
template <int MT>
__device__ __forceinline__ void gemm_block(const uint32_t (&w)[2], uint32_t q, uint32_t a2,
                                           const char* tab, const char* xbuf, uint32_t copy_off,
                                           int lane, int unit, const float* s_code2, float offset,
                                           f32x4 (&acc)[MT]) {
  const int i = lane & 15;
  // B operands: byte 4 t + e of the lane's 8 bytes holds k 16 unit + 8 t + 2 e,
  // + 1; one 8-byte table read gives its hi and lo pairs
  bf16x8 bhv[2], blv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint2 e2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t addr = __builtin_amdgcn_perm(copy_off, w[t], 0x0C0C0004u | (uint32_t(e) << 8));
      e2[e] = *reinterpret_cast<const uint2*>(tab + addr);
    }
    bhv[t] = __builtin_bit_cast(bf16x8, (u32x4){e2[0].x, e2[1].x, e2[2].x, e2[3].x});
    blv[t] = __builtin_bit_cast(bf16x8, (u32x4){e2[0].y, e2[1].y, e2[2].y, e2[3].y});
  }
  const float prod = s_code2[q & 0xFFu] * f16_to_f32(static_cast<uint16_t>(a2));
  const float a = prod + offset;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // A operands: row 16 mt + i, k 16 unit + 8 t .. + 7
    const char* row = xbuf + (16 * mt + i) * kGemmXRow + 32 * unit;
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row));
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16));
    f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, bhv[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, blv[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, bhv[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, blv[1], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] += a * c[r];
  }
}

template <int MT>
__global__ __launch_bounds__(kGemmThreads) void gemm_mfma_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ absmax_q,
    const uint16_t* __restrict__ absmax2, const uint16_t* __restrict__ code2, float offset, int M,
    int N, int K, int log2bs, int log2s2, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, float* __restrict__ part, int SK) {
  constexpr int R = gemm_r<MT>();
  constexpr int BM = 16 * MT;
  constexpr int XTILE = BM * kGemmXRow;   // LDS bytes of one block's activations
  constexpr int XGROUP = 2 * R * XTILE;   // ... of one group's
  static_assert(gemm_xloads<MT>() <= 16, "chunk offsets");
  static_assert(4 * MT * 64 * sizeof(f32x4) <= 256 * kPairCopies * sizeof(uint2),
                "the second-half sums fit in the decode table's LDS");
  __shared__ uint2 s_pairs[256 * kPairCopies];  // 64 KiB decode table
  __shared__ float s_code2[256];
  __shared__ __attribute__((aligned(16))) char s_x[2 * XGROUP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  // the unit of each block the lane row holds: its own (one block per load)
  // or the one gather_units leaves it (four blocks per load)
  const int unit = gemm_r<MT>() == 4 ? unit_of_row(g) : g;
  const int n = blockIdx.x * 64 + (wave & 3) * 16 + j;  // the lane's column
  const int m0 = blockIdx.y * BM;
  const int split = blockIdx.z;

  GemmLane L;
  const uint64_t nk = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  const uint64_t nb = ((nk - 1) >> log2bs) + 1;
  const uint64_t ng = ((nb - 1) >> log2s2) + 1;
  L.rp = rsrc(packed, static_cast<uint32_t>(nk >> 1));
  L.rq = rsrc(absmax_q, static_cast<uint32_t>(nb));
  L.ra2 = rsrc(absmax2, static_cast<uint32_t>(ng * 2));
  L.rx = rsrc(x, static_cast<uint32_t>(static_cast<uint64_t>(M) * K * 2));
  L.wrow = n < N ? static_cast<uint32_t>(n) * static_cast<uint32_t>(K >> 1) : kFar;
  L.blk_row = static_cast<uint32_t>(n < N ? n : 0) * static_cast<uint32_t>(K);
  L.g = static_cast<uint32_t>(g);
  L.half = static_cast<uint32_t>(wave >> 2);
  L.xg_live = R * MT >= 2 || tid < 256;
#pragma unroll
  for (int i = 0; i < gemm_xloads<MT>(); ++i) {
    const int c = tid + kGemmThreads * i;
    const int b = c / (128 * MT), r = (c >> 3) % (16 * MT);
    // threads without a chunk load from out of range (in the VGPR offset)
    L.xg_off[i] = static_cast<uint32_t>(m0 + r) * static_cast<uint32_t>(K) * 2u +
                  static_cast<uint32_t>(b) * 128u + static_cast<uint32_t>(c & 7) * 16u +
                  (L.xg_live ? 0u : kFar);
  }
  L.log2bs = log2bs;
  L.log2s2 = log2s2;

  // this workgroup's range of K blocks, taken in groups of 2 R from kb0
  const int nkb = K >> 6;
  const int kb0 = (split * nkb / SK) / (2 * R) * (2 * R);
  const int kb1 = split + 1 == SK ? nkb : ((split + 1) * nkb / SK) / (2 * R) * (2 * R);
  const int gp0 = kb0 / (2 * R), gp1 = (kb1 + 2 * R - 1) / (2 * R);
  constexpr int S = gemm_stages<MT>();
  GemmStage<MT> st[S];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) gemm_load<MT>(st[i], gp0 + i, kb1, L);

  if (tid < 256) s_code2[tid] = f16_to_f32(code2[tid]);
  build_pair_table(s_pairs, tid, blockDim.x);
  const uint32_t copy_off = static_cast<uint32_t>(lane % kPairCopies) * 8u;
  gemm_stash<MT>(st[0], s_x, tid);
  __syncthreads();
  const char* tab = reinterpret_cast<const char*>(s_pairs);

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // group p: its activations are in LDS buffer (p - gp0) & 1, the wave's
  // weights in st[(p - gp0) % S]; the loads of group p + S - 1 go out before it
  // is computed and group p + 1's activations are stashed after it
  // The loop runs whole rounds of S groups: every group of a round issues its
  // loads (past gp1 they are dead, out of range), stashes and meets the
  // barrier, and only the compute of blocks past kb1 is skipped.  A guard around the loads
  // instead would give the loop header paths with different numbers of loads
  // in flight, and the compiler then waits for all of them (vmcnt(0)) at the
  // top of every group, which undoes the prefetch.
  for (int gp = gp0; gp < gp1; gp += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int p = gp + u;
      gemm_load<MT>(st[(u + S - 1) % S], p + S - 1, kb1, L);
      uint32_t wl[R][2];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wl[r][0] = st[u].w[r][0];
        wl[r][1] = st[u].w[r][1];
      }
      if constexpr (R == 4) gather_units(wl);
      const char* xbuf = s_x + ((p - gp0) & 1) * XGROUP + L.half * (R * XTILE);
      const int kbw = p * 2 * R + static_cast<int>(L.half) * R;
      // (computing dead blocks too, with scale 0, measured 1.8x slower at
      // 128 rows and no faster at 16)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (kbw + r < kb1)
          gemm_block<MT>(wl[r], st[u].q[r], st[u].a2[r], tab, xbuf + r * XTILE, copy_off, lane,
                         unit, s_code2, offset, acc);
      gemm_stash<MT>(st[(u + 1) % S], s_x + ((p + 1 - gp0) & 1) * XGROUP, tid);
      __syncthreads();
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // the second-half waves' sums go to the first-half waves through the
  // table's LDS (every wave is past its last table read: the loop ends on a
  // barrier)
  f32x4* s_red = reinterpret_cast<f32x4*>(s_pairs);  // [4 waves][MT][64]
  if (wave >= 4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[((wave - 4) * MT + mt) * 64 + lane] = acc[mt];
  }
  __syncthreads();
  if (wave >= 4) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 o = s_red[(wave * MT + mt) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] += o[r];
  }
  if (n >= N) return;
  // SK == 1: the bf16 tile; else the partial tile into plane `split` of the
  // workspace (summed by gemm_reduce_kernel)
  float* dst = SK > 1 ? part + static_cast<int64_t>(split) * M * N : nullptr;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mt + 4 * g + r;
      if (m >= M) continue;
      const int64_t o = static_cast<int64_t>(m) * N + n;
      if (SK > 1)
        dst[o] = acc[mt][r];
      else
        y[o] = to_half_bits<NF4_BF16>(acc[mt][r]);
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
  p.gx = (N + 63) / 64;
  p.gy = (M + 16 * p.MT - 1) / (16 * p.MT);
  const int64_t tiles = p.gx * p.gy;
  // one workgroup per CU (LDS)
  const int64_t slots = static_cast<int64_t>(device_cus());
  const int64_t nkb = K / 64;
  p.SK = 1;
  constexpr int64_t kFixed = 8;  // per-workgroup cost in blocks
  int64_t best = ((tiles + slots - 1) / slots) * (nkb + kFixed);
  for (int sk = 2; sk <= 8; ++sk) {
    if (nkb < 8 * sk) break;  // at least a few groups of blocks per split
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
  switch (p.MT) {
#define NF4_GEMM_MT(T)                                                                          \
  case T:                                                                                       \
    hipLaunchKernelGGL((gemm_mfma_kernel<T>), grid, block, 0, st, packed, absmax_q, absmax2,   \
                       code2, offset, m, nn, k, lbs, ls2, x, y, part, p.SK);                     \
    break;
    NF4_GEMM_MT(1)
    NF4_GEMM_MT(2)
    NF4_GEMM_MT(4)
    NF4_GEMM_MT(8)
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
