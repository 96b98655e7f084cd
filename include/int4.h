/*
 * int4.h -- C ABI of the INT4 asymmetric group format in libnf4: dequant,
 * fused W4A16 GEMV and the GPU encoder, on AMD Instinct MI355X (gfx950).
 * Status codes, dtypes and all conventions (device pointers owned by the
 * caller, asynchronous work on `stream`, synchronous argument validation, no
 * allocation, thread safety) are those of nf4.h.
 *
 * Page cited (by title and section):
 *  [handbook] "量化与 GEMV" (anrans.github.io CUDA handbook): "量化公式"
 *             (asymmetric quantization with a zero point), "W4A16：在寄存器里
 *             反量化" (8 weights per 32-bit word, the first in the low 4 bits;
 *             a scale and a zero point per group of G = 128 consecutive
 *             elements; value = (q - z) * s), "GEMV kernel 的写法".
 *
 * ---------------------------------------------------------------------------
 * The format (one flattened tensor of n elements; a GEMV weight is [N][K]
 * row-major, flattened, so with K % G == 0 the groups are the page's
 * [N][K/G] per-row groups)
 * ---------------------------------------------------------------------------
 *  packed  uint8[ceil(n/2)]  codes q in 0..15; element 2i in the LOW nibble
 *                            of byte i, element 2i+1 in the HIGH nibble (the
 *                            little-endian bytes of the page's 32-bit words).
 *  scales  fp16[ceil(n/G)]   scale s of group e / G.
 *  zeros   fp16[ceil(n/G)]   zero point z of group e / G.
 *  value   = fp32(fp32(q - z) * s)   (q - z is exact in fp32)
 * G (group_size) is a power of two >= 2.
 */
#ifndef INT4_H_
#define INT4_H_

#include <stddef.h>
#include <stdint.h>

#include "nf4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * int4_dequant -- dequant of n elements to bf16 or fp16 (round to nearest
 * even), bit-exact with the value above.
 *  packed, scales, zeros : the format above (device).
 *  n, out, out_dtype, stream : as for nf4_dequant.
 *  group_size    : G, a power of two in [2, 2^30].
 * Returns NF4_EINVAL for a NULL pointer with n > 0, n < 0, a bad group size
 * or an unknown dtype; NF4_EUNSUPPORTED for n >= 2^40.
 */
nf4_status int4_dequant(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                        int64_t n, int32_t group_size, void* out, int32_t out_dtype,
                        void* stream);

/*
 * int4_gemv -- fused dequant + matrix-vector product for batch 1..8 (W4A16
 * decode): y[b][r] = sum_k value(r*K + k) * x[b][k] ([handbook] "W4A16：在寄
 * 存器里反量化" and "GEMV kernel 的写法").
 *  packed, scales, zeros : the format above for W [N][K].
 *  N, K, x, batch, y, stream : as for nf4_gemv (bf16 x and y).
 *  group_size    : G, a power of two in [2, 2^30].
 * The main kernels apply each group's zero point once per lane piece, as
 * s (sum q x - z sum x) with fp32 sums: each output is the bf16 rounding
 * (nearest even) of a value within 2^-14 sum_k (|q| + |z|) |s| |x_k| of the
 * exact sum.  Deterministic.  Returns NF4_EINVAL as nf4_gemv does.
 */
nf4_status int4_gemv(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, int32_t group_size, const uint16_t* x, int32_t batch,
                     uint16_t* y, void* stream);

/*
 * One matrix of a grouped INT4 GEMV (64 bytes, the layout of nf4_gemv_desc
 * with the scales and zero points in the second and third slots; device
 * pointers).
 */
typedef struct int4_gemv_desc {
  const uint8_t* packed;      /* packed codes of W [N][K], 16-byte aligned */
  const uint16_t* scales;     /* fp16 per group, 2-byte aligned */
  const uint16_t* zeros;      /* fp16 per group, 2-byte aligned */
  const uint16_t* x;          /* bf16 [batch][K], 16-byte aligned */
  uint16_t* y;                /* bf16 [batch][N] output */
  int64_t N;                  /* rows of W */
  int64_t row_begin;          /* sum of N over the preceding descriptors */
  float reserved1;            /* set to 0 */
  int32_t reserved2;          /* set to 0 */
} int4_gemv_desc;

/*
 * int4_gemv_grouped -- int4_gemv over a list of matrices in one launch
 * (independent products that share K, the group size and the batch), as
 * nf4_gemv_grouped does for the NF4 format.  Same arithmetic and tolerance
 * as int4_gemv.
 *  descs, count, total_rows, K, batch, sched, sched_bytes, stream : as for
 *                  nf4_gemv_grouped.
 *  group_size    : G, a power of two >= 32.
 * Returns NF4_EINVAL / NF4_EUNSUPPORTED as nf4_gemv_grouped does; a matrix
 * whose packed or x pointer is not 16-byte aligned, whose scales or zeros
 * are not 2-byte aligned, whose pointers are NULL or whose N disagrees with
 * the row_begin sequence is skipped (its y is left unwritten).
 */
nf4_status int4_gemv_grouped(const int4_gemv_desc* descs, int32_t count, int64_t total_rows,
                             int64_t K, int32_t group_size, int32_t batch, void* sched,
                             size_t sched_bytes, void* stream);

/*
 * int4_quantize -- encode n fp32 weights into the format above on the GPU
 * ([handbook] "量化公式"): per group, s = fp16(fp32(max - min) / 15), taken
 * as 1 when that is 0; z = round(-min / s) stored as fp16; q = clamp(round(w
 * / s) + z, 0, 15); round is to nearest with halves away from zero, fp32
 * arithmetic with the stored fp16 s.
 *  w             : device fp32[n].
 *  packed, scales, zeros : device outputs, sizes as above.
 * Returns NF4_EINVAL for NULL pointers (n > 0) or a bad group size;
 * NF4_EUNSUPPORTED for n >= 2^40.
 */
nf4_status int4_quantize(const float* w, int64_t n, int32_t group_size, uint8_t* packed,
                         uint16_t* scales, uint16_t* zeros, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INT4_H_ */
