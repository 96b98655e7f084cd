/*
 * nf4_oracle.c -- CPU oracle for the NF4 double-quantization path.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check of the package entry point and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or
 * constant generator with the HIP path (w4a16_gemv_amd/csrc); the two are
 * written independently and compared output by output.
 *
 * Plain, slow and obviously correct: scalar loops, integer division for the
 * block/group index, fp32 arithmetic in the order the method states (compile
 * with -ffp-contract=off so that no multiply-add is fused), fp64 for the GEMV
 * reference.  OpenMP only splits independent outputs across threads; it never
 * changes the order of an output's arithmetic.
 *
 * Sources (web pages; cited by title and section):
 *  [blog]     "NF4反量化算子优化" (roundaboutt.github.io): sections "什么是NF4量化？"
 *             (NF4 table), "双量化" (double quantization), "反量化", and the
 *             "naive" kernel section which prints the 16 table values to 8
 *             decimals.
 *  [report]   "NF4 双重量化反量化 CUDA Kernel 实现报告" (InfiniTensor
 *             Learning-CUDA, 03_nf4_dequant): §1.1 (table, 4 decimals, nibble
 *             packing), §1.2 (two-level scales: blocksize, s2_blocksize,
 *             absmax_q, absmax2 fp16, code2 fp16[256], offset fp32), §1.3
 *             (dequant formula), §2.2 step 1 (high nibble = even element).
 *  [quanttax] "RTX 4060 上的 LLM 量化实测" (akiliu.vercel.app, quantization-tax):
 *             section "Kernel 实现" (fused dequant-GEMV: fp32 scale x code,
 *             fp32 accumulation of weight x activation per output row).
 *  [handbook] "量化与 GEMV" (anrans.github.io CUDA handbook): "GEMV kernel 的写法"
 *             (y = W x, W is N x K row-major) and the gemv_w4 listing's fp64
 *             CPU reference used to separate kernel error from quantization
 *             error.
 *
 * Readings where the pages are silent or disagree (each is listed in the
 * design notes of the repository):
 *  - dequant: absmax_real = f32(f32(code2[q]) * f32(absmax2[g])) + offset,
 *    rounded to fp32 after the product and after the sum; value =
 *    f32(NF4[idx] * absmax_real); output = round-to-nearest-even to bf16/fp16.
 *  - quantizer: level-1 codes are chosen against the true fp32 block absmax;
 *    offset = f32(fp64 sum of block absmax / number of blocks), the sum taken
 *    in block-index order starting from +0 (the pages give no order; this is
 *    the plainest one, and it is fixed so that the value is reproducible);
 *    level 2 centres each block absmax by offset, takes the group max of |.|
 *    rounded to fp16 as absmax2, and picks the nearest code2 entry of
 *    centred/absmax2 (fp32).  Ties go to the smaller index.  A block whose
 *    absmax is 0 gets code index 7 (the exact zero) everywhere.
 *  - code2 (linear variant): fp16 nearest to -1 + 2 i / 255, i = 0..255.
 *  - odd n: the pad (low) nibble of the last byte is written as 0, ignored
 *    when reading.
 *  [handbook] also defines the INT4 asymmetric group format (sections
 *  "量化公式" and "W4A16：在寄存器里反量化"): see the INT4 part at the end.
 *  - single-level format ([quanttax] "量化的标准预期": one fp32 absmax per
 *    block of 64; "Kernel 实现": the fused kernel multiplies the fp32 code
 *    value by the block's fp32 scale): value = f32(NF4[idx] * absmax[block]),
 *    one rounding; the quantizer is the level-1 step of the double-quantized
 *    one (true block absmax, nearest NF4 code, ties to the smaller index).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 1

/* The 16 NF4 values as printed to 8 decimals in [blog], "naive" section; the C
 * compiler rounds each decimal literal to the nearest fp32. */
static const float NF4_TABLE[16] = {
    -1.00000000f, -0.69619280f, -0.52507305f, -0.39491749f,
    -0.28444138f, -0.18477343f, -0.09105004f, 0.00000000f,
    0.07958030f,  0.16093020f,  0.24611230f,  0.33791524f,
    0.44070983f,  0.56261700f,  0.72295684f,  1.00000000f,
};

int oracle_abi_version(void) { return ORACLE_ABI; }

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_nf4_table(float out[16]) { memcpy(out, NF4_TABLE, sizeof(NF4_TABLE)); }

/* ------------------------------------------------------------------------ */
/* IEEE binary16 / bfloat16 conversions, written from the format definitions */
/* ------------------------------------------------------------------------ */

/* Round the real number v (a double) to a binary floating-point format with
 * `mant` fraction bits, `ebits` exponent bits, minimum normal exponent `emin`
 * and maximum exponent `emax` (bias = emax); round to nearest, ties to even;
 * overflow to infinity; subnormals kept.  Returns the encoded bits (sign,
 * biased exponent, fraction). */
static uint32_t round_to_binary(double v, int mant, int ebits, int emin, int emax) {
    const int bias = emax;
    const uint32_t sgn = (signbit(v) ? 1u : 0u) << (mant + ebits);
    const uint32_t inf_bits = ((1u << ebits) - 1u) << mant;
    if (isnan(v)) return inf_bits | (1u << (mant - 1)); /* canonical quiet NaN */
    double a = fabs(v);
    if (isinf(a)) return sgn | inf_bits;
    if (a == 0.0) return sgn;
    int e2;
    frexp(a, &e2);        /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;       /* floor(log2(a)) */
    if (E < emin) E = emin; /* subnormal range: fixed quantum */
    const double q = ldexp(1.0, E - mant); /* value of one unit in the last place */
    const double m = a / q;                /* exact: division by a power of two */
    double fl = floor(m);
    const double frac = m - fl;            /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    const double one = ldexp(1.0, mant);   /* implicit leading 1 */
    if (fl >= 2.0 * one) { fl *= 0.5; E += 1; }
    if (fl < one) return sgn | (uint32_t)fl; /* subnormal (E == emin) or zero */
    if (E > emax) return sgn | inf_bits;
    return sgn | ((uint32_t)(E + bias) << mant) | (uint32_t)(fl - one);
}

/* binary16: 10 fraction bits, 5 exponent bits, normal exponents -14..15.
 * bfloat16: 7 fraction bits, 8 exponent bits, normal exponents -126..127. */
uint16_t oracle_f16_from_double(double v) { return (uint16_t)round_to_binary(v, 10, 5, -14, 15); }
uint16_t oracle_bf16_from_double(double v) { return (uint16_t)round_to_binary(v, 7, 8, -126, 127); }
uint16_t oracle_f16_from_float(float v) { return oracle_f16_from_double((double)v); }
uint16_t oracle_bf16_from_float(float v) { return oracle_bf16_from_double((double)v); }

/* Exact widening of an fp16 bit pattern. */
double oracle_f16_to_double(uint16_t h) {
    const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* Exact widening of a bf16 bit pattern. */
double oracle_bf16_to_double(uint16_t b) {
    const int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0) v = ldexp((double)m, -133);
    else if (e == 255) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 128), e - 134);
    return s ? -v : v;
}

/* Batch helpers for the tests. */
void oracle_f16_from_float_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_from_float(in[i]);
}
void oracle_bf16_from_float_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_float(in[i]);
}
void oracle_bf16_from_double_array(const double* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_double(in[i]);
}
void oracle_f16_to_double_array(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_double(in[i]);
}

/* ------------------------------------------------------------------------ */
/* code2: second-level code table                                            */
/* ------------------------------------------------------------------------ */

/* 256 evenly spaced values on [-1, 1], each the nearest fp16 of -1 + 2 i / 255
 * (computed in fp64, rounded once).  [report] §1.2 fixes code2 as fp16[256];
 * the even spacing is the workload's stated choice. */
void oracle_code2_linear(uint16_t out[256]) {
    for (int i = 0; i < 256; ++i) out[i] = oracle_f16_from_double(-1.0 + 2.0 * (double)i / 255.0);
}

/* ------------------------------------------------------------------------ */
/* Quantizer ([blog] "双量化"; [report] §1.1-1.2)                          */
/* ------------------------------------------------------------------------ */

static int nearest_nf4(float r) {
    int best = 0;
    float bestd = fabsf(r - NF4_TABLE[0]);
    for (int j = 1; j < 16; ++j) {
        const float d = fabsf(r - NF4_TABLE[j]);
        if (d < bestd) { bestd = d; best = j; }
    }
    return best;
}

static int nearest_code2(float r, const float* code2f) {
    int best = 0;
    float bestd = fabsf(r - code2f[0]);
    for (int i = 1; i < 256; ++i) {
        const float d = fabsf(r - code2f[i]);
        if (d < bestd) { bestd = d; best = i; }
    }
    return best;
}

/* Quantize fp32 weights w[0..n) (flattened) into the double-quantized NF4
 * format.  packed: ceil(n/2) bytes; absmax_q: ceil(n/bs) bytes; absmax2:
 * ceil(ceil(n/bs)/s2) fp16 values; *offset: fp32.  If block_absmax is not
 * NULL it receives the level-1 fp32 absmax per block.  Returns 0 on success. */
int oracle_quantize(const float* w, int64_t n, int32_t bs, int32_t s2, const uint16_t* code2,
                    uint8_t* packed, uint8_t* absmax_q, uint16_t* absmax2, float* offset,
                    float* block_absmax) {
    if (n < 0 || bs <= 0 || s2 <= 0) return 1;
    const int64_t nb = (n + bs - 1) / bs;
    const int64_t ng = (nb + s2 - 1) / s2;
    if (n == 0) { *offset = 0.0f; return 0; }
    float* absmax = (float*)malloc((size_t)nb * sizeof(float));
    if (!absmax) return 2;

    /* level 1: absmax of each block of bs consecutive elements */
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        float m = 0.0f;
        const int64_t e1 = (b + 1) * bs < n ? (b + 1) * bs : n;
        for (int64_t e = b * bs; e < e1; ++e) {
            const float a = fabsf(w[e]);
            if (a > m) m = a;
        }
        absmax[b] = m;
    }

    /* offset: mean of the block absmax values ([report] §1.2: one global
     * fp32 offset).  One fp64 sum in block-index order, divided by the block
     * count, rounded once to fp32. */
    double sum = 0.0;
    for (int64_t b = 0; b < nb; ++b) sum += (double)absmax[b];
    const float off = (float)(sum / (double)nb);
    *offset = off;

    float code2f[256];
    for (int i = 0; i < 256; ++i) code2f[i] = (float)oracle_f16_to_double(code2[i]);

    /* level 2: per group of s2 blocks, absmax2 = fp16(max |absmax - offset|),
     * absmax_q = nearest code2 entry of (absmax - offset) / absmax2 */
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t b0 = g * s2, b1 = (g + 1) * s2 < nb ? (g + 1) * s2 : nb;
        float gmax = 0.0f;
        for (int64_t b = b0; b < b1; ++b) {
            const float c = absmax[b] - off;
            if (fabsf(c) > gmax) gmax = fabsf(c);
        }
        absmax2[g] = oracle_f16_from_float(gmax);
        const float a2 = (float)oracle_f16_to_double(absmax2[g]);
        for (int64_t b = b0; b < b1; ++b) {
            const float c = absmax[b] - off;
            const float r = (a2 == 0.0f) ? 0.0f : c / a2;
            absmax_q[b] = (uint8_t)nearest_code2(r, code2f);
        }
    }

    /* level-1 codes: nearest NF4 value of w / absmax, two per byte, the even
     * element in the high nibble */
    const int64_t nbytes = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nbytes; ++i) {
        int idx[2] = {0, 0};
        for (int h = 0; h < 2; ++h) {
            const int64_t e = 2 * i + h;
            if (e >= n) { idx[h] = 0; continue; } /* pad nibble */
            const float m = absmax[e / bs];
            idx[h] = (m == 0.0f) ? 7 : nearest_nf4(w[e] / m);
        }
        packed[i] = (uint8_t)((idx[0] << 4) | idx[1]);
    }

    if (block_absmax) memcpy(block_absmax, absmax, (size_t)nb * sizeof(float));
    free(absmax);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequant ([report] §1.3; [blog] "反量化")                                  */
/* ------------------------------------------------------------------------ */

/* absmax_real of block `blk`: product of the two fp32-widened fp16 scales,
 * rounded to fp32, plus offset, rounded to fp32. */
static float block_scale(const uint8_t* absmax_q, const uint16_t* absmax2, const uint16_t* code2,
                         float offset, int64_t blk, int32_t s2) {
    const float c = (float)oracle_f16_to_double(code2[absmax_q[blk]]);
    const float g = (float)oracle_f16_to_double(absmax2[blk / s2]);
    const float s = c * g;
    const float a = s + offset;
    return a;
}

static int nibble_at(const uint8_t* packed, int64_t e) {
    const uint8_t byte = packed[e / 2];
    return (e % 2 == 0) ? (byte >> 4) : (byte & 15);
}

/* Unrounded fp32 dequant values for elements [e0, e1). */
void oracle_dequant_f32(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                        const uint16_t* code2, float offset, int64_t n, int32_t bs, int32_t s2,
                        int64_t e0, int64_t e1, float* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) {
        const float a = block_scale(absmax_q, absmax2, code2, offset, e / bs, s2);
        const float v = NF4_TABLE[nibble_at(packed, e)] * a;
        out[e - e0] = v;
    }
}

/* Dequant to 16-bit output for elements [e0, e1): out_dtype 0 = bf16, 1 = fp16. */
void oracle_dequant(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                    const uint16_t* code2, float offset, int64_t n, int32_t bs, int32_t s2,
                    int32_t out_dtype, int64_t e0, int64_t e1, uint16_t* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) {
        const float a = block_scale(absmax_q, absmax2, code2, offset, e / bs, s2);
        const float v = NF4_TABLE[nibble_at(packed, e)] * a;
        out[e - e0] = out_dtype == 0 ? oracle_bf16_from_float(v) : oracle_f16_from_float(v);
    }
}

/* Dequant of the elements listed in idx[0..m) (sampled checks at large n). */
void oracle_dequant_at(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                       const uint16_t* code2, float offset, int32_t bs, int32_t s2,
                       int32_t out_dtype, const int64_t* idx, int64_t m, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const int64_t e = idx[i];
        const float a = block_scale(absmax_q, absmax2, code2, offset, e / bs, s2);
        const float v = NF4_TABLE[nibble_at(packed, e)] * a;
        out[i] = out_dtype == 0 ? oracle_bf16_from_float(v) : oracle_f16_from_float(v);
    }
}

/* ------------------------------------------------------------------------ */
/* GEMV reference ([quanttax] "Kernel 实现"; [handbook] "GEMV kernel 的写法") */
/* ------------------------------------------------------------------------ */

/* y[b][r] = sum_k v[r][k] * x[b][k] in fp64, k ascending, where v is the
 * unrounded fp32 dequant value of flat element r*K + k and x is bf16.  Also
 * S[b][r] = sum_k |v[r][k] * x[b][k]| (the scale of the accumulation error).
 * rows: NULL for all N rows, else the list of nrows row indices; outputs are
 * laid out [B][nrows].  Either y or S may be NULL. */
void oracle_gemv(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                 const uint16_t* code2, float offset, int64_t N, int64_t K, int32_t bs, int32_t s2,
                 const uint16_t* x, int32_t B, const int64_t* rows, int64_t nrows,
                 double* y, double* S) {
    if (!rows) nrows = N;
    double* xd = (double*)malloc((size_t)B * (size_t)K * sizeof(double));
    if (!xd) return;
    for (int64_t i = 0; i < (int64_t)B * K; ++i) xd[i] = oracle_bf16_to_double(x[i]);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        const int64_t r = rows ? rows[j] : j;
        for (int32_t b = 0; b < B; ++b) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = r * K + k;
                const float a = block_scale(absmax_q, absmax2, code2, offset, e / bs, s2);
                const float v = NF4_TABLE[nibble_at(packed, e)] * a;
                const double p = (double)v * xd[(int64_t)b * K + k];
                acc += p;
                mag += fabs(p);
            }
            if (y) y[(int64_t)b * nrows + j] = acc;
            if (S) S[(int64_t)b * nrows + j] = mag;
        }
    }
    free(xd);
}

/* ------------------------------------------------------------------------ */
/* Single-level format: one fp32 absmax per block, no second level            */
/* ([quanttax] "量化的标准预期" and "Kernel 实现")                           */
/* ------------------------------------------------------------------------ */

/* Quantize fp32 weights w[0..n) with one fp32 absmax per block of bs
 * elements.  packed: ceil(n/2) bytes (even element in the high nibble);
 * absmax: ceil(n/bs) fp32 values.  Returns 0 on success. */
int oracle_quantize_sl(const float* w, int64_t n, int32_t bs, uint8_t* packed, float* absmax) {
    if (n < 0 || bs <= 0) return 1;
    const int64_t nb = (n + bs - 1) / bs;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        float m = 0.0f;
        const int64_t e1 = (b + 1) * bs < n ? (b + 1) * bs : n;
        for (int64_t e = b * bs; e < e1; ++e) {
            const float a = fabsf(w[e]);
            if (a > m) m = a;
        }
        absmax[b] = m;
    }
    const int64_t nbytes = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nbytes; ++i) {
        int idx[2] = {0, 0};
        for (int h = 0; h < 2; ++h) {
            const int64_t e = 2 * i + h;
            if (e >= n) continue; /* pad nibble stays 0 */
            const float m = absmax[e / bs];
            idx[h] = (m == 0.0f) ? 7 : nearest_nf4(w[e] / m);
        }
        packed[i] = (uint8_t)((idx[0] << 4) | idx[1]);
    }
    return 0;
}

/* Unrounded fp32 values of elements [e0, e1): NF4[idx] * absmax[block]. */
void oracle_dequant_sl_f32(const uint8_t* packed, const float* absmax, int64_t n, int32_t bs,
                           int64_t e0, int64_t e1, float* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) {
        const float v = NF4_TABLE[nibble_at(packed, e)] * absmax[e / bs];
        out[e - e0] = v;
    }
}

/* 16-bit output (0 = bf16, 1 = fp16) of elements [e0, e1). */
void oracle_dequant_sl(const uint8_t* packed, const float* absmax, int64_t n, int32_t bs,
                       int32_t out_dtype, int64_t e0, int64_t e1, uint16_t* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) {
        const float v = NF4_TABLE[nibble_at(packed, e)] * absmax[e / bs];
        out[e - e0] = out_dtype == 0 ? oracle_bf16_from_float(v) : oracle_f16_from_float(v);
    }
}

/* The same for the elements listed in idx[0..m). */
void oracle_dequant_sl_at(const uint8_t* packed, const float* absmax, int32_t bs,
                          int32_t out_dtype, const int64_t* idx, int64_t m, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const int64_t e = idx[i];
        const float v = NF4_TABLE[nibble_at(packed, e)] * absmax[e / bs];
        out[i] = out_dtype == 0 ? oracle_bf16_from_float(v) : oracle_f16_from_float(v);
    }
}

/* fp64 reference y[b][r] = sum_k v[r][k] * x[b][k] (k ascending) and
 * S[b][r] = sum_k |v x| for the single-level format; v is the unrounded fp32
 * value NF4[idx] * absmax[block].  Layout and arguments as oracle_gemv. */
void oracle_gemv_sl(const uint8_t* packed, const float* absmax, int64_t N, int64_t K, int32_t bs,
                    const uint16_t* x, int32_t B, const int64_t* rows, int64_t nrows, double* y,
                    double* S) {
    if (!rows) nrows = N;
    (void)N;
    double* xd = (double*)malloc((size_t)B * (size_t)K * sizeof(double));
    if (!xd) return;
    for (int64_t i = 0; i < (int64_t)B * K; ++i) xd[i] = oracle_bf16_to_double(x[i]);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        const int64_t r = rows ? rows[j] : j;
        for (int32_t b = 0; b < B; ++b) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = r * K + k;
                const float v = NF4_TABLE[nibble_at(packed, e)] * absmax[e / bs];
                const double p = (double)v * xd[(int64_t)b * K + k];
                acc += p;
                mag += fabs(p);
            }
            if (y) y[(int64_t)b * nrows + j] = acc;
            if (S) S[(int64_t)b * nrows + j] = mag;
        }
    }
    free(xd);
}

/* ------------------------------------------------------------------------ */
/* INT4 asymmetric group format ([handbook] "量化公式", "W4A16：在寄存器里  */
/* 反量化"): groups of G consecutive elements share an fp16 scale s and an   */
/* fp16 zero point z; value = (q - z) * s with q in 0..15; two codes per     */
/* byte with the FIRST (even) element in the LOW nibble.                     */
/* Readings: s = fp16(fp32(max - min) / 15), replaced by 1 when it is 0;     */
/* z = round(-min / s) and q = clamp(round(w / s) + z, 0, 15), with round    */
/* half away from zero (the page's listing rounds with std::round) in fp32,  */
/* using the stored fp16 s; z is stored as fp16; value = fp32(fp32(q - z) *  */
/* s) (the difference is exact).                                             */
/* ------------------------------------------------------------------------ */

static int int4_nibble(const uint8_t* packed, int64_t e) {
    const uint8_t byte = packed[e / 2];
    return (e % 2 == 0) ? (byte & 15) : (byte >> 4);
}

int oracle_int4_quantize(const float* w, int64_t n, int32_t G, uint8_t* packed,
                         uint16_t* scales, uint16_t* zeros) {
    if (n < 0 || G <= 0 || G % 2 != 0) return 1;  /* even G: no byte spans two groups */
    const int64_t ng = (n + G - 1) / G;
    memset(packed, 0, (size_t)((n + 1) / 2));
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t e0 = g * G, e1 = (g + 1) * G < n ? (g + 1) * G : n;
        float mn = w[e0], mx = w[e0];
        for (int64_t e = e0 + 1; e < e1; ++e) {
            if (w[e] < mn) mn = w[e];
            if (w[e] > mx) mx = w[e];
        }
        const float range = mx - mn;
        uint16_t s16 = oracle_f16_from_float(range / 15.0f);
        float s = (float)oracle_f16_to_double(s16);
        if (s == 0.0f) { s16 = oracle_f16_from_double(1.0); s = 1.0f; }
        const float zr = roundf(-mn / s);
        const uint16_t z16 = oracle_f16_from_float(zr);
        const float z = (float)oracle_f16_to_double(z16);
        scales[g] = s16;
        zeros[g] = z16;
        for (int64_t e = e0; e < e1; ++e) {
            float q = roundf(w[e] / s) + z;
            if (q < 0.0f) q = 0.0f;
            if (q > 15.0f) q = 15.0f;
            const int qi = (int)q;
            /* bytes are owned by one group: G is even, so group starts are even */
            packed[e / 2] |= (uint8_t)((e % 2 == 0) ? qi : (qi << 4));
        }
    }
    return 0;
}

static float int4_value(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                        int32_t G, int64_t e) {
    const float q = (float)int4_nibble(packed, e);
    const float z = (float)oracle_f16_to_double(zeros[e / G]);
    const float s = (float)oracle_f16_to_double(scales[e / G]);
    const float d = q - z;
    const float v = d * s;
    return v;
}

void oracle_int4_dequant_f32(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                             int64_t n, int32_t G, int64_t e0, int64_t e1, float* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) out[e - e0] = int4_value(packed, scales, zeros, G, e);
}

void oracle_int4_dequant(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                         int64_t n, int32_t G, int32_t out_dtype, int64_t e0, int64_t e1,
                         uint16_t* out) {
    if (e1 > n) e1 = n;
#pragma omp parallel for schedule(static)
    for (int64_t e = e0; e < e1; ++e) {
        const float v = int4_value(packed, scales, zeros, G, e);
        out[e - e0] = out_dtype == 0 ? oracle_bf16_from_float(v) : oracle_f16_from_float(v);
    }
}

/* fp64 reference y[b][r] = sum_k v[r][k] x[b][k] (k ascending) with v the fp32
 * value above; S[b][r] = sum_k |v x|; M[b][r] = sum_k (|q| + |z|) |s| |x|,
 * the magnitude of the terms when the zero point is applied once per group
 * (sum q x minus z sum x).  Layout as oracle_gemv; y, S or M may be NULL. */
void oracle_int4_gemv(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                      int64_t N, int64_t K, int32_t G, const uint16_t* x, int32_t B,
                      const int64_t* rows, int64_t nrows, double* y, double* S, double* M) {
    if (!rows) nrows = N;
    (void)N;
    double* xd = (double*)malloc((size_t)B * (size_t)K * sizeof(double));
    if (!xd) return;
    for (int64_t i = 0; i < (int64_t)B * K; ++i) xd[i] = oracle_bf16_to_double(x[i]);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        const int64_t r = rows ? rows[j] : j;
        for (int32_t b = 0; b < B; ++b) {
            double acc = 0.0, mag = 0.0, mz = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = r * K + k;
                const double xv = xd[(int64_t)b * K + k];
                const double p = (double)int4_value(packed, scales, zeros, G, e) * xv;
                acc += p;
                mag += fabs(p);
                const double s = oracle_f16_to_double(scales[e / G]);
                const double z = oracle_f16_to_double(zeros[e / G]);
                mz += ((double)int4_nibble(packed, e) + fabs(z)) * fabs(s) * fabs(xv);
            }
            if (y) y[(int64_t)b * nrows + j] = acc;
            if (S) S[(int64_t)b * nrows + j] = mag;
            if (M) M[(int64_t)b * nrows + j] = mz;
        }
    }
    free(xd);
}
