/*
 * nf4.h -- C ABI of libnf4: NF4 double-quantization dequant and fused
 * W4A16 dequant-GEMV for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *  [blog]     "NF4反量化算子优化" (roundaboutt.github.io): "双量化", "反量化".
 *  [report]   "NF4 双重量化反量化 CUDA Kernel 实现报告" (InfiniTensor
 *             Learning-CUDA 03_nf4_dequant): §1.1-§1.3, §2.2, §3.3.
 *  [quanttax] "RTX 4060 上的 LLM 量化实测" (akiliu.vercel.app): "Kernel 实现".
 *  [handbook] "量化与 GEMV" (anrans.github.io): "GEMV kernel 的写法".
 *
 * ---------------------------------------------------------------------------
 * The quantized tensor format (one flattened tensor of n elements)
 * ---------------------------------------------------------------------------
 *  packed    uint8[ceil(n/2)]   two 4-bit NF4 indices per byte; element 2i
 *                               in the HIGH nibble, element 2i+1 in the LOW
 *                               nibble ([report] §1.1 and §2.2 step 1).  For
 *                               odd n the low nibble of the last byte is
 *                               padding and is never read.
 *  absmax_q  uint8[ceil(n/blocksize)]          per-block index into code2.
 *  absmax2   fp16[ceil(nblocks/s2_blocksize)]  per-group second-level scale.
 *  code2     fp16[256]                          second-level code table.
 *  offset    fp32                               global offset (by value).
 * ([report] §1.2 names these arrays and their types.)
 *
 * Element e belongs to block e / blocksize and group block / s2_blocksize;
 * both sizes must be powers of two, so the library uses shifts ([report]
 * §3.3).  The dequantized value is ([report] §1.3):
 *
 *     absmax_real = fp32(fp32(code2[absmax_q[block]]) * fp32(absmax2[group]))
 *                   + offset                    (rounded to fp32 again)
 *     value       = fp32(NF4[index(e)] * absmax_real)
 *
 * with each product and the sum rounded to fp32 separately (no fused
 * multiply-add), NF4 the 16-entry table printed in [blog] "naive".
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    keeps no pointer after the call returns and allocates nothing
 *    (nf4_quantize uses a workspace the caller provides).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *    stream) and runs asynchronously; results are valid once the stream has
 *    been synchronized.  No entry point synchronizes.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is launched.  n == 0 (or N*K == 0) returns
 *    NF4_OK without launching.
 *  - Calls are thread-safe: the library holds no mutable global state.
 *  - Pointers need only natural alignment; 16-byte aligned buffers take the
 *    vectorized kernels, other alignments a slower kernel with identical bits.
 */
#ifndef NF4_H_
#define NF4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NF4_OK = 0,
  NF4_EINVAL = 1,        /* bad argument; nothing was launched */
  NF4_EUNSUPPORTED = 2,  /* valid but outside the supported range (e.g. n >= 2^40) */
  NF4_EHIP = 3           /* the HIP runtime reported an error at launch */
} nf4_status;

typedef enum { NF4_BF16 = 0, NF4_FP16 = 1 } nf4_dtype;

/* Version of this ABI (incremented on incompatible change). */
int nf4_abi_version(void);

/* Static, human-readable name of a status code. */
const char* nf4_status_string(int status);

/*
 * nf4_dequant -- standalone dequant of n elements to bf16 or fp16.
 * Defined by [report] §1.3 (formula) and [blog] "反量化".
 *
 *  packed, absmax_q, absmax2, code2, offset : the format above (device).
 *  n             : number of elements, 0 <= n < 2^40.
 *  blocksize     : elements per first-level block, power of two in [1, 2^30].
 *  s2_blocksize  : blocks per second-level group, power of two in [1, 2^30].
 *  out           : device, n 16-bit values (bf16 or fp16 bits), element
 *                  order = flat element order.  Written with round to
 *                  nearest even; -0 is kept; fp16 overflow gives +-inf.
 *  out_dtype     : NF4_BF16 or NF4_FP16.
 *  stream        : hipStream_t.
 * Returns NF4_EINVAL for a NULL pointer with n > 0, n < 0, a block size that
 * is not a power of two or out of range, or an unknown dtype.
 */
nf4_status nf4_dequant(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                       const uint16_t* code2, float offset, int64_t n, int32_t blocksize,
                       int32_t s2_blocksize, void* out, int32_t out_dtype, void* stream);

/*
 * nf4_gemv -- fused dequant + matrix-vector product for batch 1..8 (W4A16
 * decode): y[b][r] = sum_k value(r*K + k) * x[b][k].
 * Defined by [quanttax] "Kernel 实现" (decode on chip, fp32 accumulation) and
 * [handbook] "GEMV kernel 的写法" (y = W x with W of shape N x K, row-major).
 *
 *  packed, absmax_q, absmax2, code2, offset : the format above for the
 *                  N*K elements of W flattened row-major; blocks and groups
 *                  follow the flat index r*K + k (they may span rows).
 *  N, K          : output and input features; K must be even (rows start on
 *                  a byte); N*K < 2^40.
 *  blocksize, s2_blocksize : as for nf4_dequant.
 *  x             : device bf16 bits [batch][K], row-major.
 *  batch         : 1..8.
 *  y             : device bf16 bits [batch][N], row-major; each output is
 *                  the fp32 sum rounded to nearest even.
 *  stream        : hipStream_t.
 * Weights are never rounded to 16 bits: each NF4 value enters the products
 * as its exact fp32 value (one matrix at batch 3-8 with K <= 4096) or as the
 * sum of two bf16 values (within 2^-16 of its fp32 value), the block scale is
 * applied in fp32, and the sum is accumulated in fp32: each output
 * is the bf16 rounding (nearest even)
 * of a value within 2^-14 * sum_k |w x| of the exact sum, so
 * |y - exact| <= 2^-8 |exact| + (1 + 2^-8) 2^-14 sum_k |w x|.  Deterministic:
 * the summation order depends only on N, K and batch.
 * Returns NF4_EINVAL for NULL pointers with N*K > 0, N < 0, K < 0, odd K,
 * batch outside 1..8, or bad block sizes.
 */
nf4_status nf4_gemv(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                    const uint16_t* code2, float offset, int64_t N, int64_t K,
                    int32_t blocksize, int32_t s2_blocksize, const uint16_t* x, int32_t batch,
                    uint16_t* y, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Single-level format: one fp32 absmax per block, no second level
 * ---------------------------------------------------------------------------
 * The same packed codes with a plain fp32 scale per block instead of the
 * double-quantized (absmax_q, absmax2, code2, offset):
 *
 *  absmax    fp32[ceil(n/blocksize)]   scale of each block of `blocksize`
 *                                      consecutive elements (4-byte aligned)
 *  value     = fp32(NF4[index(e)] * absmax[e / blocksize])   (one rounding)
 *
 * This is the format of [quanttax] "量化的标准预期" (one fp32 absmax per
 * block of 64) and of the fused kernel in its "Kernel 实现", which multiplies
 * the fp32 code value by the block's fp32 scale.  The kernels, tolerances and
 * conventions are those of the double-quantized entry points.
 */

/*
 * nf4_dequant_absmax32 -- standalone dequant of the single-level format.
 *
 *  packed        : device, ceil(n/2) bytes (nibble order as above).
 *  absmax        : device fp32 [ceil(n/blocksize)], 4-byte aligned.
 *  n, blocksize, out, out_dtype, stream : as for nf4_dequant.
 * Returns NF4_EINVAL for a NULL pointer with n > 0, a misaligned absmax,
 * n < 0, a block size that is not a power of two in [1, 2^30], or an unknown
 * dtype; NF4_EUNSUPPORTED for n >= 2^40.
 */
nf4_status nf4_dequant_absmax32(const uint8_t* packed, const float* absmax, int64_t n,
                                int32_t blocksize, void* out, int32_t out_dtype, void* stream);

/*
 * nf4_gemv_absmax32 -- fused dequant + matrix-vector product (batch 1..8) for
 * the single-level format: y[b][r] = sum_k value(r*K + k) * x[b][k].
 *
 *  packed, absmax : the single-level format of W [N][K] flattened row-major
 *                  (blocks follow the flat index r*K + k).
 *  N, K, blocksize, x, batch, y, stream : as for nf4_gemv.
 * Same accumulation and tolerance as nf4_gemv.  Returns NF4_EINVAL as
 * nf4_gemv does, and for a misaligned absmax.
 */
nf4_status nf4_gemv_absmax32(const uint8_t* packed, const float* absmax, int64_t N, int64_t K,
                             int32_t blocksize, const uint16_t* x, int32_t batch, uint16_t* y,
                             void* stream);

/*
 * nf4_gemm -- the product for any number of batch rows (prefill and batches
 * past 8): y[m][n] = sum_k value(n*K + k) * x[m][k], m < M.  Batch growth
 * makes the product compute-bound, so it runs on the matrix cores (bf16
 * MFMA with exact products and fp32 sums).  Defined as nf4_gemv; [quanttax]
 * "Kernel 实现" and its conclusions on prefill, [handbook] batch sensitivity.
 *
 *  packed, absmax_q, absmax2, code2, offset, N, K, blocksize, s2_blocksize :
 *                  as for nf4_gemv.
 *  M             : batch rows, 0 <= M < 2^27.
 *  x             : device bf16 bits [M][K], row-major.
 *  y             : device bf16 bits [M][N], row-major.
 *  workspace     : optional DEVICE scratch buffer of workspace_bytes bytes,
 *                  256-byte aligned, any contents, or NULL.  With
 *                  nf4_gemm_workspace_size(M, N, K) bytes the product may split
 *                  K over several workgroups: their fp32 partial sums go
 *                  there and a second kernel adds them in a fixed order.  The
 *                  split changes the fp32 summation order, so results may
 *                  differ from a NULL-workspace call in the last bits (both
 *                  within the tolerance below).  Nothing is kept between
 *                  calls; calls that may overlap in time (other streams) need
 *                  separate workspaces.  Caller-owned; never freed or resized
 *                  by the library.
 *  stream        : hipStream_t.
 * The fast path needs K % 64 == 0, blocksize >= 64, packed and x
 * 16-byte aligned, N*K < 2^31 and (M + 128) K < 2^30; other shapes run the
 * GEMV over chunks of 8 rows, with the same tolerance.  Weights are never
 * rounded to 16 bits (each NF4 value enters as the sum of two bf16 values,
 * within 2^-16 of it) and sums are fp32: each output is the bf16 rounding of
 * a value within 2^-14 * sum_k |w x| of the exact sum.  Deterministic: the
 * same arguments (workspace size included) give the same bits.
 * Returns NF4_EINVAL for NULL pointers with M*N*K > 0, negative sizes, odd K,
 * bad block sizes or a workspace that is not 256-byte aligned.
 */
nf4_status nf4_gemm(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                    const uint16_t* code2, float offset, int64_t M, int64_t N, int64_t K,
                    int32_t blocksize, int32_t s2_blocksize, const uint16_t* x, uint16_t* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * nf4_gemm_workspace_size -- bytes of workspace nf4_gemm can use for an
 * M x N x K product on the current device (0: it would not split K, or the
 * shape takes the GEMV path).  Depends on the device's compute-unit count.
 */
size_t nf4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * One matrix of a grouped GEMV (64 bytes; all pointers are device pointers).
 */
typedef struct nf4_gemv_desc {
  const uint8_t* packed;      /* packed codes of W [N][K], 16-byte aligned */
  const uint8_t* absmax_q;    /* per-block code2 index */
  const uint16_t* absmax2;    /* per-group fp16 scale */
  const uint16_t* x;          /* bf16 [batch][K], 16-byte aligned */
  uint16_t* y;                /* bf16 [batch][N] output */
  int64_t N;                  /* rows of W */
  int64_t row_begin;          /* sum of N over the preceding descriptors */
  float offset;               /* fp32 offset of this tensor */
  int32_t reserved;           /* set to 0 */
} nf4_gemv_desc;

/*
 * nf4_gemv_grouped -- nf4_gemv over a list of matrices in one launch, for
 * independent products that share K, the block sizes, code2 and the batch
 * (e.g. the q/k/v or gate/up projections of a decoder layer, or a whole weight
 * sweep).  Same arithmetic and tolerance as nf4_gemv; each y is written once.
 * The launch streams the concatenated rows of all matrices through one
 * persistent grid, so the per-launch ramp-up and drain are paid once.
 *
 *  descs         : DEVICE array of `count` descriptors (8-byte aligned), built
 *                  by the caller; row_begin must be the running sum of N.
 *  count         : 1..1024 descriptors (0 is a no-op).
 *  total_rows    : sum of N over all descriptors, < 2^31.
 *  K             : input features shared by all matrices; K % 32 == 0 and
 *                  K <= 16384.
 *  blocksize     : power of two >= 32; s2_blocksize: power of two.
 *  code2         : device fp16 bits [256] shared by all matrices.
 *  batch         : 1..8.
 *  sched         : optional DEVICE scheduling workspace of sched_bytes >=
 *                  nf4_gemv_sched_size() bytes, 256-byte aligned, filled with
 *                  zeros before its first use.  With it, the rows of large
 *                  launches are handed to the waves in small chunks as they
 *                  free up (better balanced than a fixed split); each launch
 *                  returns the counters it used to zero when it completes, so
 *                  one buffer serves any number of launches on one stream.
 *                  Launches that can run at the same time (other streams)
 *                  need buffers of their own.  NULL: fixed split.  The
 *                  results are bit-identical either way.
 * Returns NF4_EINVAL for a NULL or misaligned descs / code2, odd K, bad block
 * sizes, or a misaligned / too small sched; NF4_EUNSUPPORTED outside the
 * ranges above.  The descriptors are read on the device: a matrix whose
 * packed or x pointer is not 16-byte aligned, whose pointers are NULL, or
 * whose N disagrees with the row_begin sequence is skipped (its y is left
 * unwritten).  The kernel cannot report a skipped matrix; check the table
 * with nf4_gemv_desc_check on the host before uploading it.
 */
nf4_status nf4_gemv_grouped(const nf4_gemv_desc* descs, int32_t count, int64_t total_rows,
                            int64_t K, int32_t blocksize, int32_t s2_blocksize,
                            const uint16_t* code2, int32_t batch, void* sched,
                            size_t sched_bytes, void* stream);

/*
 * nf4_gemv_sched_size -- bytes of the scheduling workspace nf4_gemv_grouped
 * takes (host function).
 */
size_t nf4_gemv_sched_size(void);

/*
 * nf4_gemv_grouped_noalloc -- nf4_gemv_grouped with chunked row scheduling and
 * no workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It allocates nothing.  The scheduling counters live in the
 * library's own scratch: a fixed array of nf4_gemv_sched_size() = 2 KiB of
 * device memory, one per GPU, which each GPU the library runs on holds until
 * the process ends.  The caller passes inputs and outputs as for
 * nf4_gemv_grouped, and the results are bit-identical to it.
 *
 *  Arguments : those of nf4_gemv_grouped without sched / sched_bytes.  The
 *              current device must be the device of `stream`.
 *  Scratch   : its device address is looked up once per device
 *              (hipGetSymbolAddress, with that device current) on the first
 *              call there.  A launch that uses the counters first clears them
 *              with a small kernel on `stream`; both kernels are only
 *              enqueued.  Every call on one GPU shares that GPU's scratch,
 *              which keeps the last call's contents: calls that overlap in
 *              time on one GPU (other streams, unordered host threads) race
 *              and may compute wrong rows.  Order them on one stream.
 *  Limits    : one scratch serves every launch size the grouped entry point
 *              accepts (up to 1024 matrices, 2^31 - 1 rows, K <= 16384, batch
 *              1..8); beyond those the call returns NF4_EUNSUPPORTED without
 *              launching, as nf4_gemv_grouped does.
 * Returns the status codes of nf4_gemv_grouped (NF4_EINVAL for bad arguments,
 * before any HIP call), and NF4_EHIP when the scratch address cannot be
 * obtained or a launch fails.
 */
nf4_status nf4_gemv_grouped_noalloc(const nf4_gemv_desc* descs, int32_t count,
                                    int64_t total_rows, int64_t K, int32_t blocksize,
                                    int32_t s2_blocksize, const uint16_t* code2, int32_t batch,
                                    void* stream);

/*
 * nf4_gemv_desc_check -- host-side check of a grouped GEMV descriptor table
 * before it is uploaded (host function, no GPU work).  The grouped kernels
 * skip a descriptor they cannot use, leaving its y unwritten, and have no way
 * to report it; this function finds exactly those descriptors.
 *
 *  descs      : HOST array of `count` descriptors for nf4_gemv_grouped /
 *               nf4_gemv_grouped_noalloc (format 0), nf4_gemv_grouped_absmax32
 *               (format 1) or int4_gemv_grouped (format 2); the three layouts
 *               are the same 64 bytes.
 *  total_rows, K : as they will be passed to the grouped call.
 *  first_bad  : optional output: the index of the first unusable descriptor,
 *               `count` when the N values do not add up to total_rows, or -1
 *               when every descriptor is usable.
 * A descriptor is usable when its packed, scale, x and y pointers are not
 * NULL (the second scale slot may be NULL in format 1), packed and x are
 * 16-byte aligned, an fp32 absmax array is 4-byte and fp16 scale / zero-point
 * arrays are 2-byte aligned, 0 <= N and N * K < 2^31, and row_begin is the
 * sum of N over the descriptors before it.
 * Returns NF4_OK when all are usable, NF4_EINVAL otherwise (also for a NULL
 * table with count > 0, negative sizes or an unknown format).
 */
nf4_status nf4_gemv_desc_check(const void* descs, int32_t count, int64_t total_rows, int64_t K,
                               int32_t format, int32_t* first_bad);

/*
 * One matrix of a grouped single-level GEMV (64 bytes, the layout of
 * nf4_gemv_desc with the fp32 absmax in the second slot; device pointers).
 */
typedef struct nf4_absmax32_gemv_desc {
  const uint8_t* packed;      /* packed codes of W [N][K], 16-byte aligned */
  const float* absmax;        /* fp32 absmax per block, 4-byte aligned */
  const void* reserved0;      /* set to NULL */
  const uint16_t* x;          /* bf16 [batch][K], 16-byte aligned */
  uint16_t* y;                /* bf16 [batch][N] output */
  int64_t N;                  /* rows of W */
  int64_t row_begin;          /* sum of N over the preceding descriptors */
  float reserved1;            /* set to 0 */
  int32_t reserved2;          /* set to 0 */
} nf4_absmax32_gemv_desc;

/*
 * nf4_gemv_grouped_absmax32 -- nf4_gemv_absmax32 over a list of matrices in
 * one launch (independent products that share K, the block size and the
 * batch), as nf4_gemv_grouped does for the double-quantized format.  Same
 * arithmetic and tolerance as nf4_gemv_absmax32.
 *  descs, count, total_rows, K, batch, sched, sched_bytes, stream : as for
 *                  nf4_gemv_grouped.
 *  blocksize     : power of two >= 32.
 * Returns NF4_EINVAL / NF4_EUNSUPPORTED as nf4_gemv_grouped does; a matrix
 * whose packed or x pointer is not 16-byte aligned, whose absmax is not
 * 4-byte aligned, whose pointers are NULL or whose N disagrees with the
 * row_begin sequence is skipped (its y is left unwritten).
 */
nf4_status nf4_gemv_grouped_absmax32(const nf4_absmax32_gemv_desc* descs, int32_t count,
                                     int64_t total_rows, int64_t K, int32_t blocksize,
                                     int32_t batch, void* sched, size_t sched_bytes,
                                     void* stream);

/*
 * nf4_code2_linear -- the linear second-level code table: out[i] = the fp16
 * nearest to -1 + 2 i / 255, i = 0..255 (host function, no GPU work).  The
 * report's §1.2 fixes code2 as fp16[256]; evenly spaced values are this
 * library's default table.
 */
void nf4_code2_linear(uint16_t out[256]);

/*
 * nf4_quantize_workspace_size -- bytes of device workspace nf4_quantize needs
 * for n elements at this blocksize (0 for n <= 0).
 */
size_t nf4_quantize_workspace_size(int64_t n, int32_t blocksize);

/*
 * nf4_quantize -- encode n fp32 weights into the format above on the GPU.
 * Follows [blog] "双量化" and [report] §1.1-§1.2: per block absmax, nearest
 * NF4 code of w / absmax (two codes per byte, even element high); the block
 * absmax values are centred by offset (their mean), grouped by s2_blocksize,
 * absmax2 = fp16 of the group's largest |centred value|, absmax_q = index of
 * the nearest code2 entry to centred / absmax2.  Ties go to the smaller
 * index; an all-zero block gets code 7 (exact zero).  The mean is one fp64
 * sum of the block absmax values in block-index order, divided by the block
 * count and rounded once to fp32: the result does not depend on the launch
 * and is bit-identical on every run.  That sum is one serial chain of adds
 * (about 2 ms per 2^18 blocks); the encoder is not meant for a timed path.
 *
 *  w             : device fp32[n] (flattened weights).
 *  code2         : device fp16 bits [256] (e.g. nf4_code2_linear uploaded).
 *  packed, absmax_q, absmax2 : device outputs, sizes as in the format above.
 *  offset        : device fp32[1] output (read it back to pass it by value to
 *                  nf4_dequant / nf4_gemv).
 *  workspace     : device scratch of at least nf4_quantize_workspace_size()
 *                  bytes, 256-byte aligned, owned by the caller.
 * Returns NF4_EINVAL on NULL pointers (n > 0), bad block sizes, a short or
 * unaligned workspace.
 */
nf4_status nf4_quantize(const float* w, int64_t n, int32_t blocksize, int32_t s2_blocksize,
                        const uint16_t* code2, uint8_t* packed, uint8_t* absmax_q,
                        uint16_t* absmax2, float* offset, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * nf4_quantize_absmax32 -- encode n fp32 weights into the single-level format
 * on the GPU: the level-1 step of nf4_quantize alone ([quanttax]
 * "量化的标准预期": one fp32 absmax per block).  absmax[b] = the largest |w|
 * of block b; each code is the nearest NF4 value of w / absmax[b] (ties to the
 * smaller index; code 7, the exact zero, for an all-zero block); two codes per
 * byte, even element high.  Bit-identical to the level-1 output of
 * nf4_quantize.
 *
 *  w             : device fp32[n].
 *  packed        : device output, ceil(n/2) bytes.
 *  absmax        : device output fp32[ceil(n/blocksize)], 4-byte aligned.
 * Returns NF4_EINVAL for NULL pointers (n > 0), a misaligned absmax or a bad
 * block size; NF4_EUNSUPPORTED for n >= 2^40.
 */
nf4_status nf4_quantize_absmax32(const float* w, int64_t n, int32_t blocksize, uint8_t* packed,
                                 float* absmax, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H_ */
