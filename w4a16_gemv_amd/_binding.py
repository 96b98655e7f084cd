"""ctypes binding of libnf4 (include/nf4.h, include/int4.h).

Argument marshalling only: every step of the dequant and GEMV runs in the HIP
kernels of libnf4.so.  Tensors must live on an AMD GPU; there is no CPU
fallback, and loading fails loudly when the library has not been built.
Work goes on torch's current stream of the tensors' device.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnf4.so")

NF4_OK, NF4_EINVAL, NF4_EUNSUPPORTED, NF4_EHIP = 0, 1, 2, 3
NF4_BF16, NF4_FP16 = 0, 1

EXPORTED = ("nf4_abi_version", "nf4_status_string", "nf4_dequant", "nf4_gemv", "nf4_gemm",
            "nf4_gemm_workspace_size",
            "nf4_dequant_absmax32", "nf4_gemv_absmax32", "nf4_gemv_grouped",
            "nf4_gemv_grouped_absmax32", "int4_gemv_grouped",
            "nf4_probe_stream_read", "nf4_probe_expand_copy",
            "nf4_gemv_sched_size", "nf4_gemv_grouped_noalloc", "nf4_gemv_desc_check",
            "nf4_code2_linear", "nf4_quantize_workspace_size",
            "nf4_quantize", "nf4_quantize_absmax32", "int4_dequant", "int4_gemv",
            "int4_quantize")

_lib = None


class NF4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


def load() -> C.CDLL:
    """Load libnf4.so (built by w4a16_gemv_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m w4a16_gemv_amd.build` "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = C.CDLL(LIB_PATH)
    p, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int32, C.c_float
    lib.nf4_abi_version.restype = C.c_int
    lib.nf4_abi_version.argtypes = []
    lib.nf4_status_string.restype = C.c_char_p
    lib.nf4_status_string.argtypes = [C.c_int]
    lib.nf4_dequant.restype = C.c_int
    lib.nf4_dequant.argtypes = [p, p, p, p, f32, i64, i32, i32, p, i32, p]
    lib.nf4_gemv.restype = C.c_int
    lib.nf4_gemv.argtypes = [p, p, p, p, f32, i64, i64, i32, i32, p, i32, p, p]
    lib.nf4_dequant_absmax32.restype = C.c_int
    lib.nf4_dequant_absmax32.argtypes = [p, p, i64, i32, p, i32, p]
    lib.nf4_gemv_absmax32.restype = C.c_int
    lib.nf4_gemv_absmax32.argtypes = [p, p, i64, i64, i32, p, i32, p, p]
    lib.nf4_gemm.restype = C.c_int
    lib.nf4_gemm.argtypes = [p, p, p, p, f32, i64, i64, i64, i32, i32, p, p, p, C.c_size_t, p]
    lib.nf4_gemm_workspace_size.restype = C.c_size_t
    lib.nf4_gemm_workspace_size.argtypes = [i64, i64, i64]
    lib.nf4_gemv_grouped.restype = C.c_int
    lib.nf4_gemv_grouped.argtypes = [p, i32, i64, i64, i32, i32, p, i32, p, C.c_size_t, p]
    lib.nf4_gemv_grouped_absmax32.restype = C.c_int
    lib.nf4_gemv_grouped_absmax32.argtypes = [p, i32, i64, i64, i32, i32, p, C.c_size_t, p]
    lib.nf4_probe_stream_read.restype = C.c_int
    lib.nf4_probe_stream_read.argtypes = [p, C.c_size_t, p, p]
    lib.nf4_probe_expand_copy.restype = C.c_int
    lib.nf4_probe_expand_copy.argtypes = [p, C.c_size_t, p, p]
    lib.int4_gemv_grouped.restype = C.c_int
    lib.int4_gemv_grouped.argtypes = [p, i32, i64, i64, i32, i32, p, C.c_size_t, p]
    lib.nf4_gemv_sched_size.restype = C.c_size_t
    lib.nf4_gemv_sched_size.argtypes = []
    lib.nf4_gemv_grouped_noalloc.restype = C.c_int
    lib.nf4_gemv_grouped_noalloc.argtypes = [p, i32, i64, i64, i32, i32, p, i32, p]
    lib.nf4_gemv_desc_check.restype = C.c_int
    lib.nf4_gemv_desc_check.argtypes = [p, i32, i64, i64, i32, C.POINTER(C.c_int32)]
    lib.nf4_code2_linear.restype = None
    lib.nf4_code2_linear.argtypes = [p]
    lib.nf4_quantize_workspace_size.restype = C.c_size_t
    lib.nf4_quantize_workspace_size.argtypes = [i64, i32]
    lib.nf4_quantize.restype = C.c_int
    lib.nf4_quantize.argtypes = [p, i64, i32, i32, p, p, p, p, p, p, C.c_size_t, p]
    lib.nf4_quantize_absmax32.restype = C.c_int
    lib.nf4_quantize_absmax32.argtypes = [p, i64, i32, p, p, p]
    lib.int4_dequant.restype = C.c_int
    lib.int4_dequant.argtypes = [p, p, p, i64, i32, p, i32, p]
    lib.int4_gemv.restype = C.c_int
    lib.int4_gemv.argtypes = [p, p, p, i64, i64, i32, p, i32, p, p]
    lib.int4_quantize.restype = C.c_int
    lib.int4_quantize.argtypes = [p, i64, i32, p, p, p, p]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nf4_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != NF4_OK:
        raise NF4Error(fn, status)


def _dev(t: torch.Tensor, name: str, dtypes, min_numel: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")
    return t.data_ptr()


_U8 = (torch.uint8,)
_HALF_BITS = (torch.float16, torch.int16, torch.uint16)
_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def format_sizes(n: int, blocksize: int, s2_blocksize: int):
    nblocks = -(-n // blocksize)
    return (n + 1) // 2, nblocks, -(-nblocks // s2_blocksize)


def nf4_dequant(packed, absmax_q, absmax2, code2, offset: float, n: int, blocksize: int = 64,
                s2_blocksize: int = 256, out: torch.Tensor | None = None,
                out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Dequantize n NF4 elements to bf16 / fp16 (returns `out`, shape [n])."""
    nbytes, nb, ng = format_sizes(int(n), int(blocksize), int(s2_blocksize))
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float16")
    if out is None:
        out = torch.empty(int(n), dtype=out_dtype, device=packed.device)
    code = NF4_BF16 if out.dtype in (torch.bfloat16,) else NF4_FP16
    if out.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out must be bfloat16 or float16")
    args = (_dev(packed, "packed", _U8, nbytes), _dev(absmax_q, "absmax_q", _U8, nb),
            _dev(absmax2, "absmax2", _HALF_BITS, ng), _dev(code2, "code2", _HALF_BITS, 256))
    po = _dev(out, "out", (out.dtype,), int(n))
    st = load().nf4_dequant(*args, C.c_float(offset), int(n), int(blocksize), int(s2_blocksize),
                            po, code, _stream(out))
    _check("nf4_dequant", st)
    return out


def nf4_gemv(packed, absmax_q, absmax2, code2, offset: float, N: int, K: int, x: torch.Tensor,
             blocksize: int = 64, s2_blocksize: int = 256,
             y: torch.Tensor | None = None) -> torch.Tensor:
    """y[b][r] = sum_k W[r][k] x[b][k] with W the NF4 tensor viewed as [N][K].

    x: bf16 [batch][K] (or [K]); returns y bf16 [batch][N] (or [N])."""
    xb, batch, y, squeeze = _gemv_io(x, N, K, y)
    nbytes, nb, ng = format_sizes(int(N) * int(K), int(blocksize), int(s2_blocksize))
    args = (_dev(packed, "packed", _U8, nbytes), _dev(absmax_q, "absmax_q", _U8, nb),
            _dev(absmax2, "absmax2", _HALF_BITS, ng), _dev(code2, "code2", _HALF_BITS, 256))
    px = _dev(xb, "x", _BF16_BITS, batch * int(K))
    py = _dev(y, "y", _BF16_BITS, batch * int(N))
    st = load().nf4_gemv(*args, C.c_float(offset), int(N), int(K), int(blocksize),
                         int(s2_blocksize), px, int(batch), py, _stream(y))
    _check("nf4_gemv", st)
    return y.view(int(N)) if squeeze and y.dim() == 2 else y


def nf4_gemm_workspace(M: int, N: int, K: int, device=None) -> torch.Tensor | None:
    """A scratch workspace for nf4_gemm of an M x N x K product on `device`
    (None when the product would not use one).  Reusable by later calls of
    the same or smaller shapes on one stream (nothing is kept between calls)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        nbytes = load().nf4_gemm_workspace_size(int(M), int(N), int(K))
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def nf4_gemm(packed, absmax_q, absmax2, code2, offset: float, N: int, K: int, x: torch.Tensor,
             blocksize: int = 64, s2_blocksize: int = 256,
             y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m][n] = sum_k W[n][k] x[m][k] for any number of rows M of x (bf16
    [M][K]); returns y bf16 [M][N].  The matrix-core path for batches past 8.

    workspace: uint8 device tensor from nf4_gemm_workspace (or None: K is not
    split, which is slower when N / 64 column tiles leave compute units idle;
    the split sums K in pieces, so the two may differ in the last bits, both
    within the same tolerance)."""
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}], got shape {tuple(x.shape)}")
    M = x.shape[0]
    nbytes, nb, ng = format_sizes(int(N) * int(K), int(blocksize), int(s2_blocksize))
    if y is None:
        y = torch.empty(M, int(N), dtype=torch.bfloat16, device=x.device)
    args = (_dev(packed, "packed", _U8, nbytes), _dev(absmax_q, "absmax_q", _U8, nb),
            _dev(absmax2, "absmax2", _HALF_BITS, ng), _dev(code2, "code2", _HALF_BITS, 256))
    px = _dev(x, "x", _BF16_BITS, M * int(K))
    py = _dev(y, "y", _BF16_BITS, M * int(N))
    pw, wbytes = None, 0
    if workspace is not None:
        pw = _dev(workspace, "workspace", _U8, 0)
        wbytes = workspace.numel()
    st = load().nf4_gemm(*args, C.c_float(offset), int(M), int(N), int(K), int(blocksize),
                         int(s2_blocksize), px, py, pw, C.c_size_t(wbytes), _stream(y))
    _check("nf4_gemm", st)
    return y


_F32 = (torch.float32,)


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Bandwidth probe: read all of src (uint8, 16-byte aligned, a multiple of
    16 bytes) once; sink is a device int32 scalar tensor."""
    _check("nf4_probe_stream_read",
           load().nf4_probe_stream_read(_dev(src, "src", _U8, 0), src.numel(),
                                        _dev(sink, "sink", (torch.int32,), 1), _stream(src)))


def probe_expand_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Bandwidth probe: read src (uint8) and write 4x its bytes to dst (uint8)."""
    if dst.numel() < 4 * src.numel():
        raise ValueError("dst must hold 4x the bytes of src")
    _check("nf4_probe_expand_copy",
           load().nf4_probe_expand_copy(_dev(src, "src", _U8, 0), src.numel(),
                                        _dev(dst, "dst", _U8, 4 * src.numel()), _stream(src)))


def _gemv_io(x: torch.Tensor, N: int, K: int, y: torch.Tensor | None):
    """Shape checks shared by the GEMV wrappers: (x as [batch][K], batch, y,
    whether to return y as 1-D)."""
    if x.dim() not in (1, 2):
        raise ValueError(f"x must be 1-D or 2-D, got shape {tuple(x.shape)}")
    squeeze = x.dim() == 1
    xb = x.unsqueeze(0) if squeeze else x
    batch = xb.shape[0]
    if xb.shape[1] != K:
        raise ValueError(f"x width {xb.shape[1]} does not match K={K}")
    if not 1 <= batch <= 8:
        raise ValueError(f"batch must be 1..8, got {batch}")
    if y is None:
        y = torch.empty(batch, int(N), dtype=torch.bfloat16, device=x.device)
    return xb, batch, y, squeeze


def nf4_dequant_absmax32(packed, absmax, n: int, blocksize: int = 64,
                         out: torch.Tensor | None = None,
                         out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Dequantize n elements of the single-level format (fp32 absmax per
    block) to bf16 / fp16 (returns `out`, shape [n])."""
    nbytes = (int(n) + 1) // 2
    nb = -(-int(n) // int(blocksize))
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float16")
    if out is None:
        out = torch.empty(int(n), dtype=out_dtype, device=packed.device)
    if out.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out must be bfloat16 or float16")
    code = NF4_BF16 if out.dtype == torch.bfloat16 else NF4_FP16
    pp = _dev(packed, "packed", _U8, nbytes)
    pa = _dev(absmax, "absmax", _F32, nb)
    po = _dev(out, "out", (out.dtype,), int(n))
    st = load().nf4_dequant_absmax32(pp, pa, int(n), int(blocksize), po, code, _stream(out))
    _check("nf4_dequant_absmax32", st)
    return out


def nf4_gemv_absmax32(packed, absmax, N: int, K: int, x: torch.Tensor, blocksize: int = 64,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """y[b][r] = sum_k W[r][k] x[b][k] for W in the single-level format viewed
    as [N][K].  x: bf16 [batch][K] (or [K]); returns y bf16 [batch][N] (or [N])."""
    xb, batch, y, squeeze = _gemv_io(x, N, K, y)
    n = int(N) * int(K)
    pp = _dev(packed, "packed", _U8, (n + 1) // 2)
    pa = _dev(absmax, "absmax", _F32, -(-n // int(blocksize)))
    px = _dev(xb, "x", _BF16_BITS, batch * int(K))
    py = _dev(y, "y", _BF16_BITS, batch * int(N))
    st = load().nf4_gemv_absmax32(pp, pa, int(N), int(K), int(blocksize), px, int(batch), py,
                                  _stream(y))
    _check("nf4_gemv_absmax32", st)
    return y.view(int(N)) if squeeze and y.dim() == 2 else y


def nf4_code2_linear() -> torch.Tensor:
    """The linear code2 table (CPU int16 tensor of fp16 bit patterns)."""
    out = torch.empty(256, dtype=torch.int16)
    load().nf4_code2_linear(out.data_ptr())
    return out


class NF4Tensor:
    """A flattened tensor in the double-quantized NF4 format, on the GPU."""

    def __init__(self, packed, absmax_q, absmax2, code2, offset: float, n: int,
                 blocksize: int = 64, s2_blocksize: int = 256):
        self.packed, self.absmax_q, self.absmax2, self.code2 = packed, absmax_q, absmax2, code2
        self.offset, self.n = float(offset), int(n)
        self.blocksize, self.s2_blocksize = int(blocksize), int(s2_blocksize)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.packed, self.absmax_q, self.absmax2, self.code2)) + 4

    def dequant(self, out=None, out_dtype=torch.bfloat16):
        return nf4_dequant(self.packed, self.absmax_q, self.absmax2, self.code2, self.offset,
                           self.n, self.blocksize, self.s2_blocksize, out, out_dtype)

    def gemv(self, N: int, K: int, x, y=None):
        if N * K != self.n:
            raise ValueError(f"N*K={N * K} does not match the tensor's {self.n} elements")
        return nf4_gemv(self.packed, self.absmax_q, self.absmax2, self.code2, self.offset, N, K,
                        x, self.blocksize, self.s2_blocksize, y)

    def gemm(self, N: int, K: int, x, y=None, workspace=None):
        if N * K != self.n:
            raise ValueError(f"N*K={N * K} does not match the tensor's {self.n} elements")
        return nf4_gemm(self.packed, self.absmax_q, self.absmax2, self.code2, self.offset, N, K,
                        x, self.blocksize, self.s2_blocksize, y, workspace)


def nf4_quantize(w: torch.Tensor, blocksize: int = 64, s2_blocksize: int = 256,
                 code2: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 sync_offset: bool = True):
    """Encode fp32 weights (any shape, flattened) into an NF4Tensor on w's GPU.

    With sync_offset (default) the fp32 offset is read back to the host (one
    stream synchronization); otherwise NF4Tensor.offset is NaN and the device
    value is returned as a second result."""
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    n = w.numel()
    nbytes, nb, ng = format_sizes(n, int(blocksize), int(s2_blocksize))
    devc = w.device
    if code2 is None:
        code2 = nf4_code2_linear().to(devc)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=devc)
    absmax_q = torch.empty(nb, dtype=torch.uint8, device=devc)
    absmax2 = torch.empty(ng, dtype=torch.int16, device=devc)
    off = torch.zeros(1, dtype=torch.float32, device=devc)
    need = int(load().nf4_quantize_workspace_size(n, int(blocksize)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=devc)
    wc = w.contiguous().view(-1)
    st = load().nf4_quantize(_dev(wc, "w", (torch.float32,), n), n, int(blocksize),
                             int(s2_blocksize), _dev(code2, "code2", _HALF_BITS, 256),
                             packed.data_ptr(), absmax_q.data_ptr(), absmax2.data_ptr(),
                             off.data_ptr(), workspace.data_ptr(), workspace.numel(),
                             _stream(wc))
    _check("nf4_quantize", st)
    if sync_offset:
        return NF4Tensor(packed, absmax_q, absmax2, code2, off.item(), n, blocksize, s2_blocksize)
    return NF4Tensor(packed, absmax_q, absmax2, code2, float("nan"), n, blocksize,
                     s2_blocksize), off


class NF4Absmax32Tensor:
    """A flattened tensor in the single-level NF4 format (one fp32 absmax per
    block), on the GPU."""

    def __init__(self, packed, absmax, n: int, blocksize: int = 64):
        self.packed, self.absmax = packed, absmax
        self.n, self.blocksize = int(n), int(blocksize)

    @property
    def nbytes(self) -> int:
        return self.packed.numel() + 4 * self.absmax.numel()

    def dequant(self, out=None, out_dtype=torch.bfloat16):
        return nf4_dequant_absmax32(self.packed, self.absmax, self.n, self.blocksize, out=out,
                                    out_dtype=out_dtype)

    def gemv(self, N: int, K: int, x, y=None):
        if N * K != self.n:
            raise ValueError(f"N*K = {N * K} does not match the tensor's {self.n} elements")
        return nf4_gemv_absmax32(self.packed, self.absmax, N, K, x, self.blocksize, y=y)


def nf4_quantize_absmax32(w: torch.Tensor, blocksize: int = 64) -> NF4Absmax32Tensor:
    """Encode fp32 weights (any shape, flattened) into the single-level format
    on w's GPU."""
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    n = w.numel()
    wc = w.contiguous().view(-1)
    packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
    absmax = torch.empty(-(-n // int(blocksize)), dtype=torch.float32, device=w.device)
    st = load().nf4_quantize_absmax32(_dev(wc, "w", (torch.float32,), n), n, int(blocksize),
                                      packed.data_ptr(), absmax.data_ptr(), _stream(wc))
    _check("nf4_quantize_absmax32", st)
    return NF4Absmax32Tensor(packed, absmax, n, blocksize)


def int4_dequant(packed, scales, zeros, n: int, group_size: int = 128,
                 out: torch.Tensor | None = None,
                 out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Dequantize n elements of the INT4 asymmetric group format (include/int4.h)
    to bf16 / fp16 (returns `out`, shape [n])."""
    ng = -(-int(n) // int(group_size))
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float16")
    if out is None:
        out = torch.empty(int(n), dtype=out_dtype, device=packed.device)
    if out.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out must be bfloat16 or float16")
    code = NF4_BF16 if out.dtype == torch.bfloat16 else NF4_FP16
    pp = _dev(packed, "packed", _U8, (int(n) + 1) // 2)
    ps = _dev(scales, "scales", _HALF_BITS, ng)
    pz = _dev(zeros, "zeros", _HALF_BITS, ng)
    po = _dev(out, "out", (out.dtype,), int(n))
    st = load().int4_dequant(pp, ps, pz, int(n), int(group_size), po, code, _stream(out))
    _check("int4_dequant", st)
    return out


def int4_gemv(packed, scales, zeros, N: int, K: int, x: torch.Tensor, group_size: int = 128,
              y: torch.Tensor | None = None) -> torch.Tensor:
    """y[b][r] = sum_k W[r][k] x[b][k] for W in the INT4 asymmetric group format
    viewed as [N][K].  x: bf16 [batch][K] (or [K]); returns y bf16 [batch][N]."""
    xb, batch, y, squeeze = _gemv_io(x, N, K, y)
    n = int(N) * int(K)
    ng = -(-n // int(group_size))
    pp = _dev(packed, "packed", _U8, (n + 1) // 2)
    ps = _dev(scales, "scales", _HALF_BITS, ng)
    pz = _dev(zeros, "zeros", _HALF_BITS, ng)
    px = _dev(xb, "x", _BF16_BITS, batch * int(K))
    py = _dev(y, "y", _BF16_BITS, batch * int(N))
    st = load().int4_gemv(pp, ps, pz, int(N), int(K), int(group_size), px, int(batch), py,
                          _stream(y))
    _check("int4_gemv", st)
    return y.view(int(N)) if squeeze and y.dim() == 2 else y


class Int4Tensor:
    """A flattened tensor in the INT4 asymmetric group format, on the GPU."""

    def __init__(self, packed, scales, zeros, n: int, group_size: int = 128):
        self.packed, self.scales, self.zeros = packed, scales, zeros
        self.n, self.group_size = int(n), int(group_size)

    @property
    def nbytes(self) -> int:
        return self.packed.numel() + 2 * self.scales.numel() + 2 * self.zeros.numel()

    def dequant(self, out=None, out_dtype=torch.bfloat16):
        return int4_dequant(self.packed, self.scales, self.zeros, self.n, self.group_size,
                            out=out, out_dtype=out_dtype)

    def gemv(self, N: int, K: int, x, y=None):
        if N * K != self.n:
            raise ValueError(f"N*K = {N * K} does not match the tensor's {self.n} elements")
        return int4_gemv(self.packed, self.scales, self.zeros, N, K, x, self.group_size, y=y)


def int4_quantize(w: torch.Tensor, group_size: int = 128) -> Int4Tensor:
    """Encode fp32 weights (any shape, flattened) into the INT4 asymmetric group
    format on w's GPU."""
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    n = w.numel()
    wc = w.contiguous().view(-1)
    ng = -(-n // int(group_size))
    packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
    scales = torch.empty(ng, dtype=torch.int16, device=w.device)
    zeros = torch.empty(ng, dtype=torch.int16, device=w.device)
    st = load().int4_quantize(_dev(wc, "w", (torch.float32,), n), n, int(group_size),
                              packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), _stream(wc))
    _check("int4_quantize", st)
    return Int4Tensor(packed, scales, zeros, n, group_size)


# layout of nf4_gemv_desc (include/nf4.h), 64 bytes
_DESC_DTYPE = [("packed", "<u8"), ("absmax_q", "<u8"), ("absmax2", "<u8"), ("x", "<u8"),
               ("y", "<u8"), ("N", "<i8"), ("row_begin", "<i8"), ("offset", "<f4"),
               ("reserved", "<i4")]
MAX_GROUP = 1024


class GemvGroup:
    """A reusable list of independent GEMVs y_i = W_i x_i launched as one
    grouped call: nf4_gemv_grouped for NF4Tensor items, nf4_gemv_grouped_absmax32
    for NF4Absmax32Tensor items, int4_gemv_grouped for Int4Tensor items (one
    format per group).  All W_i share K, the block (group) size and the batch
    (1..8), and for NF4Tensor code2 too.  The descriptor table is built and
    uploaded once; launch() only enqueues the kernel (so it can be captured in
    a HIP graph).

    items: list of (w, N, x: bf16 [batch][K] tensor, y: bf16 [batch][N] tensor).
    dynamic: give the launch a scheduling workspace (owned by the group), so
    that rows go to the waves in chunks as they free up; False: fixed split.
    The results are bit-identical either way.  The group's workspace serves
    one launch at a time: do not run the same group on two streams at once.
    noalloc: NF4Tensor items only; launch through nf4_gemv_grouped_noalloc,
    which schedules rows in chunks with the library's own per-GPU scratch
    (no workspace tensor; launches on one GPU must not overlap in time).
    The table is checked on the host by nf4_gemv_desc_check before upload.

    A group of one matrix with fewer rows than 1024 per compute unit launches
    through the format's single-matrix entry point (nf4_gemv,
    nf4_gemv_absmax32, int4_gemv): its kernels take the descriptor as a kernel
    argument, so their first weight loads do not wait for the descriptor
    table to be read from memory (0.3-1 us per launch at batch 1-2), and at
    batch 3-8 one matrix runs faster on the single-matrix team kernel than on
    the grouped shared-activation kernel (11008 x 4096: 11.8 / 12.8 / 20.0 us
    against 15.7 / 17.3 / 26.0 us at batch 3 / 4 / 8).  Groups of two or more
    matrices stay one grouped launch, which is faster than their single
    launches at every batch (2 x 11008 x 4096 at batch 8: 39.3 against
    42.5 us; 3 x 4096 x 4096: 26.3 against 30.2 us).  Such a group's
    results come from the single-matrix kernels, within the same tolerance
    (the bits can differ from a grouped launch of the same matrix).
    """

    def __init__(self, items, K: int, dynamic: bool = True, noalloc: bool = False):
        import numpy as np
        if not 1 <= len(items) <= MAX_GROUP:
            raise ValueError(f"a group holds 1..{MAX_GROUP} matrices")
        self.K = int(K)
        self.items = list(items)
        w0 = items[0][0]
        self.kind = type(w0)
        if self.kind not in (NF4Tensor, NF4Absmax32Tensor, Int4Tensor):
            raise ValueError(f"unsupported tensor type {self.kind.__name__}")
        if self.kind is Int4Tensor:
            self.blocksize, self.s2_blocksize, self.code2 = w0.group_size, None, None
        elif self.kind is NF4Absmax32Tensor:
            self.blocksize, self.s2_blocksize, self.code2 = w0.blocksize, None, None
        else:
            self.blocksize, self.s2_blocksize, self.code2 = w0.blocksize, w0.s2_blocksize, w0.code2
        self.batch = items[0][2].shape[0] if items[0][2].dim() == 2 else 1
        if not 1 <= self.batch <= 8:
            raise ValueError("grouped GEMV supports batch 1..8")
        if K % 32 or K <= 0 or K > 16384:
            raise ValueError("grouped GEMV needs K % 32 == 0 and 0 < K <= 16384")
        if self.blocksize < 32:
            raise ValueError("grouped GEMV needs a block (group) size >= 32")
        table = np.zeros(len(items), dtype=np.dtype(_DESC_DTYPE))
        row = 0
        for i, (w, N, x, y) in enumerate(items):
            if type(w) is not self.kind:
                raise ValueError(f"item {i}: one tensor format per group")
            if w.n != N * K:
                raise ValueError(f"item {i}: tensor has {w.n} elements, expected {N}x{K}")
            xb = x if x.dim() == 2 else x.unsqueeze(0)
            if xb.shape != (self.batch, K):
                raise ValueError(f"item {i}: x must be [{self.batch}, {K}]")
            px = _dev(xb, "x", _BF16_BITS, self.batch * K)
            py = _dev(y, "y", _BF16_BITS, self.batch * N)
            nblk = -(-w.n // self.blocksize)
            if self.kind is Int4Tensor:
                if w.group_size != self.blocksize:
                    raise ValueError(f"item {i}: group size differs from the group's")
                pp = _dev(w.packed, "packed", _U8, (w.n + 1) // 2)
                ps = _dev(w.scales, "scales", _HALF_BITS, nblk)
                pz = _dev(w.zeros, "zeros", _HALF_BITS, nblk)
                entry = (pp, ps, pz, px, py, N, row, 0.0, 0)
            elif self.kind is NF4Absmax32Tensor:
                if w.blocksize != self.blocksize:
                    raise ValueError(f"item {i}: block size differs from the group's")
                pp = _dev(w.packed, "packed", _U8, (w.n + 1) // 2)
                pa = _dev(w.absmax, "absmax", _F32, nblk)
                entry = (pp, pa, 0, px, py, N, row, 0.0, 0)
            else:
                if (w.blocksize, w.s2_blocksize) != (self.blocksize, self.s2_blocksize):
                    raise ValueError(f"item {i}: block sizes differ from the group's")
                if w.code2.data_ptr() != self.code2.data_ptr() and not torch.equal(w.code2, self.code2):
                    raise ValueError(f"item {i}: code2 differs from the group's")
                nbytes, nb, ng = format_sizes(w.n, w.blocksize, w.s2_blocksize)
                pp = _dev(w.packed, "packed", _U8, nbytes)
                entry = (pp, _dev(w.absmax_q, "absmax_q", _U8, nb),
                         _dev(w.absmax2, "absmax2", _HALF_BITS, ng), px, py, N, row, w.offset, 0)
            if pp % 16 or px % 16:
                raise ValueError(f"item {i}: packed and x must be 16-byte aligned")
            table[i] = entry
            row += N
        self.total_rows = row
        fmt = 2 if self.kind is Int4Tensor else 1 if self.kind is NF4Absmax32Tensor else 0
        bad = C.c_int32(-1)
        st = load().nf4_gemv_desc_check(table.ctypes.data, len(items), row, self.K, fmt,
                                        C.byref(bad))
        if st != NF4_OK:
            raise ValueError(f"descriptor {bad.value} is not usable by the grouped kernels")
        dev = items[0][0].packed.device
        self.table = torch.from_numpy(table.view(np.uint8)).to(dev)
        if self.code2 is not None:
            _dev(self.code2, "code2", _HALF_BITS, 256)
        self.noalloc = bool(noalloc)
        if self.noalloc and self.kind is not NF4Tensor:
            raise ValueError("noalloc grouped launches take NF4Tensor items only")
        # below 1024 rows per compute unit: chunked scheduling (64 rows per
        # wave of a full grid of two 512-lane workgroups per compute unit)
        # would not start, and the single-matrix kernels are faster
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self.single = None
        if len(self.items) == 1 and not self.noalloc and self.total_rows < 64 * 16 * cus:
            self.single = self.items[0]
        self.sched = None
        if dynamic and not self.noalloc and self.single is None:
            nbytes = int(load().nf4_gemv_sched_size())
            self.sched = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=dev)
            if self.sched.data_ptr() % 256:
                raise RuntimeError("scheduling workspace is not 256-byte aligned")

    def launch(self) -> None:
        if self.single is not None:
            w, N, x, y = self.single
            w.gemv(N, self.K, x, y)
            return
        sp, sn = (self.sched.data_ptr(), self.sched.numel() * 4) if self.sched is not None else (None, 0)
        lib = load()
        if self.kind is Int4Tensor:
            name = "int4_gemv_grouped"
            st = lib.int4_gemv_grouped(self.table.data_ptr(), len(self.items), self.total_rows,
                                       self.K, self.blocksize, self.batch, sp, sn,
                                       _stream(self.table))
        elif self.kind is NF4Absmax32Tensor:
            name = "nf4_gemv_grouped_absmax32"
            st = lib.nf4_gemv_grouped_absmax32(self.table.data_ptr(), len(self.items),
                                               self.total_rows, self.K, self.blocksize,
                                               self.batch, sp, sn, _stream(self.table))
        elif self.noalloc:
            name = "nf4_gemv_grouped_noalloc"
            st = lib.nf4_gemv_grouped_noalloc(self.table.data_ptr(), len(self.items),
                                              self.total_rows, self.K, self.blocksize,
                                              self.s2_blocksize, self.code2.data_ptr(),
                                              self.batch, _stream(self.table))
        else:
            name = "nf4_gemv_grouped"
            st = lib.nf4_gemv_grouped(self.table.data_ptr(), len(self.items), self.total_rows,
                                      self.K, self.blocksize, self.s2_blocksize,
                                      self.code2.data_ptr(), self.batch, sp, sn,
                                      _stream(self.table))
        _check(name, st)
