"""CPU oracle for the NF4 double-quantization path, the single-level
fp32-absmax format and the INT4 asymmetric group format (ctypes wrapper).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only tests/, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import this package.
It shares no code with the HIP path in w4a16_gemv_amd/ and does not import it.

The arithmetic lives in nf4_oracle.c (plain scalar C, fp32 in the method's
order without contraction, fp64 GEMV); this module only marshals numpy arrays.
Sources and readings are listed in the C file's header.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16 = 0
FP16 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    p = C.c_void_p
    i64, i32, f32 = C.c_int64, C.c_int32, C.c_float
    sig = {
        "oracle_abi_version": (C.c_int, []),
        "oracle_set_threads": (None, [C.c_int]),
        "oracle_max_threads": (C.c_int, []),
        "oracle_nf4_table": (None, [p]),
        "oracle_f16_from_double": (C.c_uint16, [C.c_double]),
        "oracle_bf16_from_double": (C.c_uint16, [C.c_double]),
        "oracle_f16_to_double": (C.c_double, [C.c_uint16]),
        "oracle_bf16_to_double": (C.c_double, [C.c_uint16]),
        "oracle_f16_from_float_array": (None, [p, i64, p]),
        "oracle_bf16_from_float_array": (None, [p, i64, p]),
        "oracle_f16_to_double_array": (None, [p, i64, p]),
        "oracle_bf16_from_double_array": (None, [p, i64, p]),
        "oracle_code2_linear": (None, [p]),
        "oracle_quantize": (C.c_int, [p, i64, i32, i32, p, p, p, p, p, p]),
        "oracle_dequant_f32": (None, [p, p, p, p, f32, i64, i32, i32, i64, i64, p]),
        "oracle_dequant": (None, [p, p, p, p, f32, i64, i32, i32, i32, i64, i64, p]),
        "oracle_dequant_at": (None, [p, p, p, p, f32, i32, i32, i32, p, i64, p]),
        "oracle_gemv": (None, [p, p, p, p, f32, i64, i64, i32, i32, p, i32, p, i64, p, p]),
        "oracle_quantize_sl": (C.c_int, [p, i64, i32, p, p]),
        "oracle_dequant_sl_f32": (None, [p, p, i64, i32, i64, i64, p]),
        "oracle_dequant_sl": (None, [p, p, i64, i32, i32, i64, i64, p]),
        "oracle_dequant_sl_at": (None, [p, p, i32, i32, p, i64, p]),
        "oracle_gemv_sl": (None, [p, p, i64, i64, i32, p, i32, p, i64, p, p]),
        "oracle_int4_quantize": (C.c_int, [p, i64, i32, p, p, p]),
        "oracle_int4_dequant_f32": (None, [p, p, p, i64, i32, i64, i64, p]),
        "oracle_int4_dequant": (None, [p, p, p, i64, i32, i32, i64, i64, p]),
        "oracle_int4_gemv": (None, [p, p, p, i64, i64, i32, p, i32, p, i64, p, p, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def nf4_table() -> np.ndarray:
    out = np.empty(16, np.float32)
    _load().oracle_nf4_table(_ptr(out))
    return out


def code2_linear() -> np.ndarray:
    out = np.empty(256, np.uint16)
    _load().oracle_code2_linear(_ptr(out))
    return out


def f16_from_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_f16_from_float_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_bf16_from_float_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_from_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bits of fp64 values, rounded once (nearest, ties to even)."""
    a = np.ascontiguousarray(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_bf16_from_double_array(_ptr(a), a.size, _ptr(out))
    return out


def f16_to_f64(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().oracle_f16_to_double_array(_ptr(h), h.size, _ptr(out))
    return out


def f16_from_f64_scalar(v: float) -> int:
    return int(_load().oracle_f16_from_double(float(v)))


def bf16_to_f64_scalar(b: int) -> float:
    return float(_load().oracle_bf16_to_double(int(b)))


@dataclass
class Quantized:
    """The double-quantized NF4 format of one flattened tensor of n elements."""
    packed: np.ndarray      # uint8 [ceil(n/2)], even element in the high nibble
    absmax_q: np.ndarray    # uint8 [ceil(n/blocksize)], index into code2
    absmax2: np.ndarray     # uint16 fp16 bits [ceil(nblocks/s2_blocksize)]
    code2: np.ndarray       # uint16 fp16 bits [256]
    offset: float           # fp32
    n: int
    blocksize: int = 64
    s2_blocksize: int = 256
    block_absmax: np.ndarray | None = None  # fp32 level-1 absmax (quantizer side info)

    @property
    def nblocks(self) -> int:
        return (self.n + self.blocksize - 1) // self.blocksize

    @property
    def ngroups(self) -> int:
        return (self.nblocks + self.s2_blocksize - 1) // self.s2_blocksize


def quantize(w: np.ndarray, blocksize: int = 64, s2_blocksize: int = 256,
             code2: np.ndarray | None = None, keep_absmax: bool = False) -> Quantized:
    w = np.ascontiguousarray(w, np.float32).reshape(-1)
    n = w.size
    if code2 is None:
        code2 = code2_linear()
    code2 = np.ascontiguousarray(code2, np.uint16)
    nb = (n + blocksize - 1) // blocksize
    ng = (nb + s2_blocksize - 1) // s2_blocksize
    packed = np.empty((n + 1) // 2, np.uint8)
    absmax_q = np.empty(nb, np.uint8)
    absmax2 = np.empty(ng, np.uint16)
    off = np.zeros(1, np.float32)
    babs = np.empty(nb, np.float32) if keep_absmax else None
    rc = _load().oracle_quantize(_ptr(w), n, blocksize, s2_blocksize, _ptr(code2), _ptr(packed),
                                 _ptr(absmax_q), _ptr(absmax2), _ptr(off), _ptr(babs))
    if rc != 0:
        raise RuntimeError(f"oracle_quantize failed: {rc}")
    return Quantized(packed, absmax_q, absmax2, code2, float(off[0]), n, blocksize, s2_blocksize,
                     babs)


def _qargs(q: Quantized):
    return (_ptr(q.packed), _ptr(q.absmax_q), _ptr(q.absmax2), _ptr(q.code2), C.c_float(q.offset))


def dequant_f32(q: Quantized, e0: int = 0, e1: int | None = None) -> np.ndarray:
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.float32)
    _load().oracle_dequant_f32(*_qargs(q), q.n, q.blocksize, q.s2_blocksize, e0, e1, _ptr(out))
    return out


def dequant(q: Quantized, out_dtype: int = BF16, e0: int = 0, e1: int | None = None) -> np.ndarray:
    """16-bit output bits (uint16) of elements [e0, e1)."""
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.uint16)
    _load().oracle_dequant(*_qargs(q), q.n, q.blocksize, q.s2_blocksize, int(out_dtype), e0, e1,
                           _ptr(out))
    return out


def dequant_at(q: Quantized, idx: np.ndarray, out_dtype: int = BF16) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.uint16)
    _load().oracle_dequant_at(*_qargs(q), q.blocksize, q.s2_blocksize, int(out_dtype), _ptr(idx),
                              idx.size, _ptr(out))
    return out


def gemv(q: Quantized, N: int, K: int, x_bf16: np.ndarray, rows: np.ndarray | None = None):
    """fp64 reference y = W x (and S = |W| |x|) for W = q viewed as [N][K].

    x_bf16: uint16 bf16 bits [B][K].  Returns (y, S) as float64 [B][len(rows) or N].
    """
    assert N * K == q.n
    x = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, K)
    B = x.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = rows.size
    else:
        nr = N
    y = np.empty((B, nr), np.float64)
    S = np.empty((B, nr), np.float64)
    _load().oracle_gemv(*_qargs(q), N, K, q.blocksize, q.s2_blocksize, _ptr(x), B, _ptr(rows),
                        nr, _ptr(y), _ptr(S))
    return y, S


@dataclass
class QuantizedSL:
    """The single-level NF4 format: one fp32 absmax per block, no second level."""
    packed: np.ndarray      # uint8 [ceil(n/2)], even element in the high nibble
    absmax: np.ndarray      # float32 [ceil(n/blocksize)]
    n: int
    blocksize: int = 64

    @property
    def nblocks(self) -> int:
        return (self.n + self.blocksize - 1) // self.blocksize


def quantize_sl(w: np.ndarray, blocksize: int = 64) -> QuantizedSL:
    w = np.ascontiguousarray(w, np.float32).reshape(-1)
    n = w.size
    packed = np.empty((n + 1) // 2, np.uint8)
    absmax = np.empty((n + blocksize - 1) // blocksize, np.float32)
    rc = _load().oracle_quantize_sl(_ptr(w), n, blocksize, _ptr(packed), _ptr(absmax))
    if rc != 0:
        raise RuntimeError(f"oracle_quantize_sl failed: {rc}")
    return QuantizedSL(packed, absmax, n, blocksize)


def dequant_sl_f32(q: QuantizedSL, e0: int = 0, e1: int | None = None) -> np.ndarray:
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.float32)
    _load().oracle_dequant_sl_f32(_ptr(q.packed), _ptr(q.absmax), q.n, q.blocksize, e0, e1,
                                  _ptr(out))
    return out


def dequant_sl(q: QuantizedSL, out_dtype: int = BF16, e0: int = 0,
               e1: int | None = None) -> np.ndarray:
    """16-bit output bits (uint16) of elements [e0, e1)."""
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.uint16)
    _load().oracle_dequant_sl(_ptr(q.packed), _ptr(q.absmax), q.n, q.blocksize, int(out_dtype),
                              e0, e1, _ptr(out))
    return out


def dequant_sl_at(q: QuantizedSL, idx: np.ndarray, out_dtype: int = BF16) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.uint16)
    _load().oracle_dequant_sl_at(_ptr(q.packed), _ptr(q.absmax), q.blocksize, int(out_dtype),
                                 _ptr(idx), idx.size, _ptr(out))
    return out


def gemv_sl(q: QuantizedSL, N: int, K: int, x_bf16: np.ndarray,
            rows: np.ndarray | None = None):
    """fp64 reference (y, S) for the single-level format; as gemv()."""
    assert N * K == q.n
    x = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, K)
    B = x.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = rows.size
    else:
        nr = N
    y = np.empty((B, nr), np.float64)
    S = np.empty((B, nr), np.float64)
    _load().oracle_gemv_sl(_ptr(q.packed), _ptr(q.absmax), N, K, q.blocksize, _ptr(x), B,
                           _ptr(rows), nr, _ptr(y), _ptr(S))
    return y, S


@dataclass
class QuantizedInt4:
    """The INT4 asymmetric group format: codes 0..15 (first element of each
    byte in the LOW nibble), one fp16 scale and one fp16 zero point per group
    of G consecutive elements."""
    packed: np.ndarray      # uint8 [ceil(n/2)]
    scales: np.ndarray      # uint16 fp16 bits [ceil(n/G)]
    zeros: np.ndarray       # uint16 fp16 bits [ceil(n/G)]
    n: int
    group: int = 128


def int4_quantize(w: np.ndarray, group: int = 128) -> QuantizedInt4:
    w = np.ascontiguousarray(w, np.float32).reshape(-1)
    n = w.size
    ng = -(-n // group)
    packed = np.empty((n + 1) // 2, np.uint8)
    scales = np.empty(ng, np.uint16)
    zeros = np.empty(ng, np.uint16)
    rc = _load().oracle_int4_quantize(_ptr(w), n, group, _ptr(packed), _ptr(scales), _ptr(zeros))
    if rc != 0:
        raise RuntimeError(f"oracle_int4_quantize failed: {rc}")
    return QuantizedInt4(packed, scales, zeros, n, group)


def _i4args(q: QuantizedInt4):
    return (_ptr(q.packed), _ptr(q.scales), _ptr(q.zeros))


def int4_dequant_f32(q: QuantizedInt4, e0: int = 0, e1: int | None = None) -> np.ndarray:
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.float32)
    _load().oracle_int4_dequant_f32(*_i4args(q), q.n, q.group, e0, e1, _ptr(out))
    return out


def int4_dequant(q: QuantizedInt4, out_dtype: int = BF16, e0: int = 0,
                 e1: int | None = None) -> np.ndarray:
    e1 = q.n if e1 is None else min(e1, q.n)
    out = np.empty(max(e1 - e0, 0), np.uint16)
    _load().oracle_int4_dequant(*_i4args(q), q.n, q.group, int(out_dtype), e0, e1, _ptr(out))
    return out


def int4_gemv(q: QuantizedInt4, N: int, K: int, x_bf16: np.ndarray,
              rows: np.ndarray | None = None):
    """fp64 reference (y, S, M) for W = q viewed as [N][K]: S = sum |w x| and
    M = sum (|q| + |z|) |s| |x| (the magnitude of the terms when the zero point
    is applied once per group)."""
    assert N * K == q.n
    x = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, K)
    B = x.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = rows.size
    else:
        nr = N
    y = np.empty((B, nr), np.float64)
    S = np.empty((B, nr), np.float64)
    M = np.empty((B, nr), np.float64)
    _load().oracle_int4_gemv(*_i4args(q), N, K, q.group, _ptr(x), B, _ptr(rows), nr, _ptr(y),
                             _ptr(S), _ptr(M))
    return y, S, M
