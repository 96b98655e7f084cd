"""Helpers for the GPU parity tests: move oracle-format arrays to the device,
read 16-bit results back, guard buffers and the GEMV tolerance rule."""
import numpy as np
import torch

GUARD = 64                 # guard elements on each side of an output buffer
GUARD_BITS = 0xA5A5


def dev():
    return torch.device("cuda:0")


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev())


def h16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(dev())


def fmt_to_device(q):
    return dict(packed=u8(q.packed), absmax_q=u8(q.absmax_q), absmax2=h16(q.absmax2),
                code2=h16(q.code2))


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def guarded(n: int, dtype: torch.dtype, offset_elems: int = 0):
    """A buffer of n elements (returned as a view) with GUARD_BITS-filled guard
    regions before and after it; `offset_elems` shifts the view to make it
    unaligned."""
    base = torch.full((n + 2 * GUARD + offset_elems,), GUARD_BITS - 65536, dtype=torch.int16,
                      device=dev())
    view = base[GUARD + offset_elems: GUARD + offset_elems + n].view(dtype)
    return base, view


def guards_intact(base: torch.Tensor, n: int, offset_elems: int = 0) -> bool:
    b = bits16(base)
    lo = b[: GUARD + offset_elems]
    hi = b[GUARD + offset_elems + n:]
    return bool(np.all(lo == GUARD_BITS) and np.all(hi == GUARD_BITS))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def x_to_device(xbits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(xbits, np.uint16).view(np.int16)).to(dev()) \
        .view(torch.bfloat16)


S_TOL = 2.0 ** -14


def gemv_bounds(y_ref: np.ndarray, S: np.ndarray):
    """The bf16 values a correct kernel may return: the bf16 rounding (nearest
    even) of any real within 2^-14 * S of the fp64 result, S = sum_k |w x|.
    2^-14 * S covers fp32 accumulation in any order with up to ~1000
    sequential additions per partial sum (worst case (n - 1) 2^-24 S); the
    rounding of y to bf16 (8 significant bits, up to 2^-8 relative) is taken
    exactly.  Returns (lo, hi) as float64 arrays."""
    import oracle
    d = S_TOL * S
    lo = bf16_to_f64(oracle.bf16_from_f64(y_ref - d))
    hi = bf16_to_f64(oracle.bf16_from_f64(y_ref + d))
    return lo, hi


def gemv_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray):
    """Returns (ok, worst) where worst is the largest |y - y_ref| divided by the
    implied bound 2^-8 |y_ref| + (1 + 2^-8) 2^-14 S (a number <= 1 when ok)."""
    lo, hi = gemv_bounds(y_ref, S)
    ok = bool(np.all((y_gpu >= lo) & (y_gpu <= hi)))
    bound = 2.0 ** -8 * np.abs(y_ref) + (1 + 2.0 ** -8) * S_TOL * S
    err = np.abs(y_gpu - y_ref)
    worst = float(np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1), 0))) \
        if err.size else 0.0
    return ok, worst


ONE_HOT_REL = 2.0 ** -15


def one_hot_ok(y: np.ndarray, w_col: np.ndarray) -> bool:
    """For x = e_k the GEMV output of row r is a single product: the kernels
    that decode through the bf16 pair table feed each NF4 value as the sum of
    two bf16 values (within 2^-16 of its fp32 value), times the block scale
    in fp32.  So y[r] must be the bf16 rounding (nearest even) of a real
    within 2^-15 |W[r][k]| of the fp32 weight W[r][k] -- far tighter than one
    bf16 step, so a wrong row, column or batch index still fails."""
    import oracle
    w = w_col.astype(np.float64)
    d = ONE_HOT_REL * np.abs(w)
    lo = bf16_to_f64(oracle.bf16_from_f64(w - d))
    hi = bf16_to_f64(oracle.bf16_from_f64(w + d))
    return bool(np.all((y >= lo) & (y <= hi)))
