"""w4a16_gemv_amd: NF4 double-quantization dequant and fused W4A16 GEMV for
AMD Instinct MI355X (gfx950).

The compute lives in libnf4.so (HIP, C ABI in include/nf4.h); this package is
its Python binding.  See nf4_dequant / nf4_gemv (double-quantized format) and
nf4_dequant_absmax32 / nf4_gemv_absmax32 (one fp32 absmax per block), and
int4_dequant / int4_gemv (INT4 asymmetric groups, include/int4.h); nf4_gemm
is the matrix-core product for batches past 8.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    GemvGroup,
    Int4Tensor,
    LIB_PATH,
    NF4Absmax32Tensor,
    NF4_BF16,
    NF4_EHIP,
    NF4_EINVAL,
    NF4_EUNSUPPORTED,
    NF4_FP16,
    NF4_OK,
    NF4Error,
    NF4Tensor,
    format_sizes,
    int4_dequant,
    int4_gemv,
    int4_quantize,
    load,
    nf4_code2_linear,
    nf4_dequant,
    nf4_dequant_absmax32,
    nf4_gemm,
    nf4_gemm_workspace,
    nf4_gemv,
    nf4_gemv_absmax32,
    nf4_quantize,
    nf4_quantize_absmax32,
    probe_expand_copy,
    probe_stream_read,
    status_string,
)
