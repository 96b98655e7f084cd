"""ctypes binding of libnf4 (include/nf4.h).

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

EXPORTED = ("nf4_abi_version", "nf4_status_string", "nf4_dequant", "nf4_gemv")

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
    if x.dim() not in (1, 2):
        raise ValueError(f"x must be 1-D or 2-D, got shape {tuple(x.shape)}")
    squeeze = x.dim() == 1
    xb = x.unsqueeze(0) if squeeze else x
    batch = xb.shape[0]
    if xb.shape[1] != K:
        raise ValueError(f"x width {xb.shape[1]} does not match K={K}")
    if not 1 <= batch <= 8:
        raise ValueError(f"batch must be 1..8, got {batch}")
    nbytes, nb, ng = format_sizes(int(N) * int(K), int(blocksize), int(s2_blocksize))
    if y is None:
        y = torch.empty(batch, int(N), dtype=torch.bfloat16, device=x.device)
    args = (_dev(packed, "packed", _U8, nbytes), _dev(absmax_q, "absmax_q", _U8, nb),
            _dev(absmax2, "absmax2", _HALF_BITS, ng), _dev(code2, "code2", _HALF_BITS, 256))
    px = _dev(xb, "x", _BF16_BITS, batch * int(K))
    py = _dev(y, "y", _BF16_BITS, batch * int(N))
    st = load().nf4_gemv(*args, C.c_float(offset), int(N), int(K), int(blocksize),
                         int(s2_blocksize), px, int(batch), py, _stream(y))
    _check("nf4_gemv", st)
    return y.view(int(N)) if squeeze and y.dim() == 2 else y
