"""Pins for the CPU oracle (no GPU needed).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden), closed forms, exact rational arithmetic, library
conversions (numpy float16, torch bfloat16, numpy float64 matmul) and brute
force on tiny inputs.  A plausible slip anywhere in the oracle -- a wrong table
entry, swapped nibbles, a dropped offset, a fused multiply-add, a wrong
block/group index, a truncating conversion, a transposed GEMV -- fails at least
one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# ----------------------------------------------------------------------------
# helpers independent of the oracle
# ----------------------------------------------------------------------------


def round_fraction(x: Fraction, mant: int = 23, emin: int = -126) -> Fraction:
    """Exact round-to-nearest-even of a rational to a binary format with `mant`
    fraction bits (default: IEEE single), no overflow handling."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # floor(log2(a)) by integer bit lengths, then fix up
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - mant)
    m = a / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def f16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def bf16_bits_torch(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def f16_bits_numpy(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):   # overflow to +-inf is the expected result
        return np.ascontiguousarray(a, np.float32).astype(np.float16).view(np.uint16)


def make_q(packed, absmax_q, absmax2, code2, offset, n, bs, s2):
    return oracle.Quantized(np.ascontiguousarray(packed, np.uint8),
                            np.ascontiguousarray(absmax_q, np.uint8),
                            np.ascontiguousarray(absmax2, np.uint16),
                            np.ascontiguousarray(code2, np.uint16),
                            float(np.float32(offset)), n, bs, s2)


@pytest.fixture(scope="module")
def page_table(nf4_literals_8dp):
    return np.array([np.float32(v) for v in nf4_literals_8dp], np.float32)


# ----------------------------------------------------------------------------
# NF4 table
# ----------------------------------------------------------------------------


def test_nf4_table_equals_blog_literals(page_table):
    t = oracle.nf4_table()
    assert t.view(np.uint32).tolist() == page_table.view(np.uint32).tolist()


def test_nf4_table_rounds_to_report_values(nf4_literals_4dp):
    # the two pages print the same table at different precisions
    t = oracle.nf4_table()
    for i, s in enumerate(nf4_literals_4dp):
        assert round(float(t[i]), 4) == pytest.approx(float(s), abs=1e-12), i


def test_nf4_table_invariants():
    t = oracle.nf4_table()
    assert t.view(np.uint32)[7] == 0          # exactly +0
    assert t[0] == -1.0 and t[15] == 1.0      # endpoints
    assert np.all(np.diff(t) > 0)             # strictly increasing
    assert (t < 0).sum() == 7 and (t > 0).sum() == 8


def test_largest_nf4_gap():
    t = oracle.nf4_table().astype(np.float64)
    gaps = np.diff(t)
    assert int(np.argmax(gaps)) == 0          # between -1 and the next code
    assert gaps.max() == pytest.approx(0.3038072, abs=1e-7)


# ----------------------------------------------------------------------------
# 16-bit conversions
# ----------------------------------------------------------------------------

EDGE_F32 = np.array([
    0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, -65520.0, 65536.0, 1e30, -1e30,
    2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -15,
    1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
    1.0 + 2.0 ** -8 + 2.0 ** -20, 3.3895314e38, 3.4028235e38, 1e-40, -1e-45, 1e-38,
    np.inf, -np.inf, 0.1, -0.3, 1234.5678,
], np.float32)


def _random_f32(n, seed):
    bits = np.random.default_rng(seed).integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_fp16_rne_matches_numpy():
    with np.errstate(over="ignore"):
        for a in (EDGE_F32, _random_f32(1_000_000, 11),
                  np.random.default_rng(12).standard_normal(200_000).astype(np.float32) * 1e3):
            assert np.array_equal(oracle.f16_from_f32(a), f16_bits_numpy(a))


def test_bf16_rne_matches_torch():
    for a in (EDGE_F32, _random_f32(1_000_000, 13)):
        assert np.array_equal(oracle.bf16_from_f32(a), bf16_bits_torch(a))


def test_bf16_from_f64_is_correctly_rounded():
    """fp64 -> bf16 rounds once: checked against exact rational rounding."""
    rng = np.random.default_rng(14)
    v = rng.standard_normal(3000) * 2.0 ** rng.integers(-140, 120, 3000)
    v = np.concatenate([v, [1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8,
                            -(1 + 2.0 ** -8 - 2.0 ** -45), 2.0 ** -133, 2.0 ** -134,
                            3 * 2.0 ** -135]])
    got = oracle.bf16_from_f64(v)
    for val, b in zip(v, got):
        exp = round_fraction(Fraction(float(val)), mant=7, emin=-126)
        gotv = Fraction(oracle.bf16_to_f64_scalar(int(b)))
        assert gotv == exp, (val, b)


def test_fp16_decode_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(h)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.all(np.isinf(got[np.isinf(ref)])) and np.all(np.isnan(got[np.isnan(ref)]))


def test_bf16_decode_matches_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64_scalar(int(v)) for v in b[::37]])
    r = ref[::37]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])


# ----------------------------------------------------------------------------
# code2
# ----------------------------------------------------------------------------


def test_code2_linear_is_nearest_fp16_of_even_grid():
    c = oracle.code2_linear()
    vals = c.view(np.float16).astype(np.float64)
    assert vals[0] == -1.0 and vals[255] == 1.0
    assert np.all(np.diff(vals) > 0)
    for i in range(256):
        target = Fraction(-1) + Fraction(2 * i, 255)
        here = Fraction(float(vals[i]))
        up = Fraction(float(np.nextafter(np.float16(vals[i]), np.float16(2))))
        dn = Fraction(float(np.nextafter(np.float16(vals[i]), np.float16(-2))))
        assert abs(here - target) <= abs(up - target) and abs(here - target) <= abs(dn - target)


# ----------------------------------------------------------------------------
# dequant
# ----------------------------------------------------------------------------

F16_ONE = 0x3C00


def test_exhaustive_byte_decode(page_table):
    """All 256 packed bytes with absmax_real = 1: the even element is the high
    nibble, the odd element the low nibble (NF4 report §2.2, step 1)."""
    code2 = np.zeros(256, np.uint16)
    code2[200] = F16_ONE
    packed = np.arange(256, dtype=np.uint8)
    q = make_q(packed, np.full(8, 200, np.uint8), np.array([F16_ONE], np.uint16), code2, 0.0,
               512, 64, 256)
    v = oracle.dequant_f32(q)
    expect = np.empty(512, np.float32)
    expect[0::2] = page_table[np.arange(256) >> 4]
    expect[1::2] = page_table[np.arange(256) & 15]
    assert np.array_equal(v.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("n,bs,s2", [(4096, 64, 4), (1000, 64, 4), (777, 32, 2), (65, 64, 256),
                                     (2, 64, 256), (64 * 256 * 3 + 64, 64, 256), (300, 2, 8),
                                     (513, 128, 2)])
def test_dequant_index_math_closed_form(n, bs, s2):
    """code2[i] = i, absmax2[g] = 2^g, offset = 1/2 and every code = 15 (value
    1): element e must read exactly absmax_q[e // bs] * 2^((e // bs) // s2) + 1/2."""
    nb = (n + bs - 1) // bs
    ng = (nb + s2 - 1) // s2
    code2 = np.arange(256, dtype=np.float32).astype(np.float16).view(np.uint16)
    absmax2 = (2.0 ** (np.arange(ng) % 12)).astype(np.float16).view(np.uint16)
    rng = np.random.default_rng(n)
    absmax_q = rng.integers(0, 256, nb).astype(np.uint8)
    packed = np.full((n + 1) // 2, 0xFF, np.uint8)
    q = make_q(packed, absmax_q, absmax2, code2, 0.5, n, bs, s2)
    v = oracle.dequant_f32(q).astype(np.float64)
    e = np.arange(n)
    blk = e // bs
    expect = absmax_q[blk].astype(np.float64) * 2.0 ** ((blk // s2) % 12) + 0.5
    assert np.array_equal(v, expect)
    # code 0 is -1 and code 7 is +0 times the same scale
    q0 = make_q(np.zeros_like(packed), absmax_q, absmax2, code2, 0.5, n, bs, s2)
    assert np.array_equal(oracle.dequant_f32(q0).astype(np.float64), -expect)
    q7 = make_q(np.full_like(packed, 0x77), absmax_q, absmax2, code2, 0.5, n, bs, s2)
    assert np.all(oracle.dequant_f32(q7).view(np.uint32) == 0)


def _random_format(rng, n, bs, s2):
    nb = (n + bs - 1) // bs
    ng = (nb + s2 - 1) // s2
    packed = rng.integers(0, 256, (n + 1) // 2).astype(np.uint8)
    absmax_q = rng.integers(0, 256, nb).astype(np.uint8)
    # fp16 scales spread over many binades, including subnormals and negatives
    a2 = (rng.standard_normal(ng) * 2.0 ** rng.integers(-20, 8, ng)).astype(np.float16)
    code2 = (rng.standard_normal(256) * 2.0 ** rng.integers(-6, 3, 256)).astype(np.float16)
    off = np.float32(rng.standard_normal() * 0.05)
    return packed, absmax_q, a2.view(np.uint16), code2.view(np.uint16), off


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dequant_matches_exact_rational(seed, page_table):
    """Brute force in exact rationals: product rounded to fp32, plus offset
    rounded to fp32, times the NF4 value rounded to fp32; then the 16-bit
    outputs equal numpy's (fp16) and torch's (bf16) RNE casts of that value."""
    rng = np.random.default_rng(100 + seed)
    n, bs, s2 = 1501, 64, 4
    packed, absmax_q, absmax2, code2, off = _random_format(rng, n, bs, s2)
    q = make_q(packed, absmax_q, absmax2, code2, off, n, bs, s2)
    got = oracle.dequant_f32(q)
    offF = Fraction(float(off))
    expect = np.empty(n, np.float32)
    for e in range(n):
        blk = e // bs
        c = f16_value(int(code2[absmax_q[blk]]))
        g = f16_value(int(absmax2[blk // s2]))
        a = round_fraction(round_fraction(c * g) + offF)
        byte = int(packed[e // 2])
        nib = byte >> 4 if e % 2 == 0 else byte & 15
        prod = round_fraction(Fraction(float(page_table[nib])) * a)
        if prod == 0:   # IEEE: +0 times a negative scale is -0
            prod_f = np.float32(-0.0) if a < 0 else np.float32(0.0)
        else:
            prod_f = np.float32(float(prod))
        expect[e] = prod_f
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
    assert np.array_equal(oracle.dequant(q, oracle.BF16), bf16_bits_torch(expect))
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle.dequant(q, oracle.FP16), f16_bits_numpy(expect))


def test_dequant_special_cases(page_table):
    n, bs, s2 = 640, 64, 4
    rng = np.random.default_rng(7)
    packed = rng.integers(0, 256, n // 2).astype(np.uint8)
    nib = np.empty(n, np.int64)
    nib[0::2] = packed >> 4
    nib[1::2] = packed & 15
    nb, ng = n // bs, (n // bs + s2 - 1) // s2
    absmax_q = rng.integers(0, 256, nb).astype(np.uint8)
    code2 = oracle.code2_linear()
    # absmax2 = 0: only the offset survives
    off = np.float32(0.0371)
    q = make_q(packed, absmax_q, np.zeros(ng, np.uint16), code2, off, n, bs, s2)
    assert np.array_equal(oracle.dequant_f32(q), page_table[nib] * off)
    # offset = 0, code2 = +-1, absmax2 = power of two: plain two-level product
    c2 = np.where(np.arange(256) < 128, -1.0, 1.0).astype(np.float16).view(np.uint16)
    a2 = (2.0 ** -np.arange(1, ng + 1)).astype(np.float16).view(np.uint16)
    q = make_q(packed, absmax_q, a2, c2, 0.0, n, bs, s2)
    blk = np.arange(n) // bs
    sgn = np.where(absmax_q[blk] < 128, -1.0, 1.0)
    expect = page_table[nib].astype(np.float64) * sgn * 2.0 ** -((blk // s2) + 1)
    assert np.array_equal(oracle.dequant_f32(q).astype(np.float64), expect)
    # a negative absmax_real turns the zero code into -0
    c2n = np.full(256, 0xBC00, np.uint16)  # -1
    q = make_q(np.full(n // 2, 0x77, np.uint8), absmax_q, np.full(ng, F16_ONE, np.uint16), c2n,
               0.0, n, bs, s2)
    assert np.all(oracle.dequant_f32(q).view(np.uint32) == 0x80000000)
    assert np.all(oracle.dequant(q, oracle.BF16) == 0x8000)
    assert np.all(oracle.dequant(q, oracle.FP16) == 0x8000)


def test_dequant_sampled_and_ranges_agree():
    w = synth.weights(5, 10_000)
    q = oracle.quantize(w)
    full = oracle.dequant(q, oracle.FP16)
    idx = np.random.default_rng(0).integers(0, q.n, 500)
    assert np.array_equal(oracle.dequant_at(q, idx, oracle.FP16), full[idx])
    assert np.array_equal(oracle.dequant(q, oracle.FP16, 1234, 5678), full[1234:5678])


# ----------------------------------------------------------------------------
# quantizer
# ----------------------------------------------------------------------------


def _nibbles(q):
    nib = np.empty(2 * q.packed.size, np.int64)
    nib[0::2] = q.packed >> 4
    nib[1::2] = q.packed & 15
    return nib[: q.n]


@pytest.mark.parametrize("n,bs,s2,seed", [(4096, 64, 4, 1), (3001, 64, 8, 2), (255, 32, 2, 3),
                                          (64 * 256 + 5, 64, 256, 4)])
def test_quantizer_brute_force(n, bs, s2, seed, page_table):
    w = synth.weights(seed, n, outliers=True)
    q = oracle.quantize(w, bs, s2, keep_absmax=True)
    nb = (n + bs - 1) // bs
    wp = np.concatenate([w, np.zeros(nb * bs - n, np.float32)]).reshape(nb, bs)
    absmax = np.abs(wp).max(axis=1)
    assert np.array_equal(q.block_absmax, absmax)
    assert q.offset == pytest.approx(math.fsum(absmax.astype(np.float64)) / nb, rel=2 ** -23)
    off = np.float32(q.offset)
    c = absmax - off
    code2f = q.code2.view(np.float16).astype(np.float32)
    for g in range(q.ngroups):
        cg = c[g * s2:(g + 1) * s2]
        a2 = np.float32(np.abs(cg).max()).astype(np.float16)
        assert q.absmax2[g] == a2.view(np.uint16)
        a2f = np.float32(a2)
        r = cg / a2f if a2f != 0 else np.zeros_like(cg)
        d = np.abs(r[:, None] - code2f[None, :])   # fp32 distances
        assert np.array_equal(q.absmax_q[g * s2:(g + 1) * s2], np.argmin(d, axis=1))
    r = w / np.repeat(absmax, bs)[:n]
    d = np.abs(r[:, None] - page_table[None, :])
    assert np.array_equal(_nibbles(q), np.argmin(d, axis=1))
    if n % 2:
        assert q.packed[-1] & 15 == 0   # pad nibble


def test_quantizer_roundtrip_bound():
    """|w - NF4[idx] * absmax| <= half the largest gap * absmax, and at the
    value level the double-quantized scale adds |absmax - absmax_real|."""
    w = synth.weights(21, 1 << 16, outliers=True)
    q = oracle.quantize(w, keep_absmax=True)
    t = oracle.nf4_table().astype(np.float64)
    half_gap = np.diff(t).max() / 2
    absmax = np.repeat(q.block_absmax, 64)[: q.n].astype(np.float64)
    lvl1 = t[_nibbles(q)] * absmax
    assert np.all(np.abs(w - lvl1) <= half_gap * absmax * (1 + 2 ** -20))
    v = oracle.dequant_f32(q).astype(np.float64)
    a_real = np.abs(v / np.where(t[_nibbles(q)] == 0, np.nan, t[_nibbles(q)]))
    a_real = np.where(np.isnan(a_real), absmax, a_real)
    bound = half_gap * a_real + np.abs(absmax - a_real) + 1e-7
    assert np.all(np.abs(w - v) <= bound)


def test_quantizer_gridpoints_are_stable():
    rng = np.random.default_rng(9)
    t = oracle.nf4_table()
    nb = 200
    A = np.float32(0.01) + rng.random(nb, dtype=np.float32)
    j = rng.integers(0, 16, (nb, 64))
    j[:, 0] = 15                      # every block holds +A, so its absmax is A
    w = (t[j] * A[:, None]).astype(np.float32).reshape(-1)
    q = oracle.quantize(w)
    assert np.array_equal(_nibbles(q), j.reshape(-1))


def test_quantizer_ties_go_to_smaller_index():
    """Where the fp32 midpoint of two neighbouring codes is an exact tie in fp32
    distance, the smaller index wins."""
    t = oracle.nf4_table()
    ties = []
    for j in range(15):
        mid = np.float32((np.float64(t[j]) + np.float64(t[j + 1])) / 2)
        if abs(mid - t[j]) == abs(mid - t[j + 1]):
            ties.append((j, mid))
    assert len(ties) >= 4
    w = np.zeros(64, np.float32)
    w[0] = 1.0                      # block absmax 1: w / absmax == w
    for i, (j, mid) in enumerate(ties):
        w[1 + i] = mid
    q = oracle.quantize(w)
    assert [int(v) for v in _nibbles(q)[1:1 + len(ties)]] == [j for j, _ in ties]


def test_quantizer_zero_tensor():
    q = oracle.quantize(np.zeros(1000, np.float32))
    assert np.all(q.packed == 0x77)
    assert np.all(oracle.dequant_f32(q) == 0.0)
    assert q.offset == 0.0 and np.all(q.absmax2 == 0)


def _blocks_with_absmax(a, bs=64):
    """Weights whose block b holds the single non-zero a[b] (so its absmax is
    exactly a[b])."""
    w = np.zeros((len(a), bs), np.float32)
    w[:, 0] = np.asarray(a, np.float32)
    return w.reshape(-1)


def test_quantizer_offset_is_the_index_order_fp64_mean():
    """offset = fp32(fp64 sum of the block absmax values in block order / nb).
    Hand-derived cases (2048 blocks, so the division by nb is exact) where the
    summation order shows in the fp32 result; the exact mean, a reverse-order
    sum and per-1024-block partial sums all give the other answer in case 1.

    Case 1: blocks 0, 1 = 1, 2^-24; blocks 1024-1026 = 2^-54; the rest 0.  In
    block order 1 + 2^-24 is exact and each 2^-54 is a quarter of the fp64
    ulp of 1, so it is lost: the sum is 1 + 2^-24 and the mean
    2^-11 + 2^-35 is the midpoint of two fp32 neighbours, which rounds to
    even, 2^-11.  Summed exactly (or the three 2^-54 first) the mean is
    above the midpoint and rounds up to 2^-11 + 2^-34.

    Case 2: blocks 0-2 = 2^-54 first, then 1 and 2^-24.  3 * 2^-54 is exact,
    adding 1 rounds it up to one fp64 ulp (2^-52), so the sum is
    1 + 2^-24 + 2^-52 and the mean rounds up to 2^-11 + 2^-34."""
    a = np.zeros(2048)
    a[0], a[1], a[1024:1027] = 1.0, 2.0 ** -24, 2.0 ** -54
    q = oracle.quantize(_blocks_with_absmax(a))
    assert np.float32(q.offset) == np.float32(2.0 ** -11)
    b = np.zeros(2048)
    b[0:3], b[3], b[4] = 2.0 ** -54, 1.0, 2.0 ** -24
    q = oracle.quantize(_blocks_with_absmax(b))
    assert np.float32(q.offset) == np.float32(2.0 ** -11 + 2.0 ** -34)
    assert np.float32(2.0 ** -11 + 2.0 ** -34) != np.float32(2.0 ** -11)


# ----------------------------------------------------------------------------
# GEMV reference
# ----------------------------------------------------------------------------


def test_gemv_one_hot_reproduces_columns():
    N, K = 48, 256
    q = oracle.quantize(synth.weights(3, N * K), 64, 4)
    W = oracle.dequant_f32(q).reshape(N, K)
    for k in (0, 1, 63, 64, 200, 255):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, S = oracle.gemv(q, N, K, synth.to_bf16_bits(x))
        assert np.array_equal(y[0], W[:, k].astype(np.float64))
        assert np.array_equal(S[0], np.abs(W[:, k]).astype(np.float64))


@pytest.mark.parametrize("N,K,B", [(64, 512, 1), (33, 1536, 4), (7, 128, 8), (20, 256, 33)])
def test_gemv_matches_float64_matmul(N, K, B):
    q = oracle.quantize(synth.weights(N + K, N * K), 64, 8)
    W = oracle.dequant_f32(q).reshape(N, K).astype(np.float64)
    xb = synth.activations(7, B, K)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    y, S = oracle.gemv(q, N, K, xb)
    assert np.allclose(y, xf @ W.T, rtol=1e-12, atol=1e-12 * np.abs(xf) @ np.abs(W).T)
    assert np.allclose(S, np.abs(xf) @ np.abs(W).T, rtol=1e-12)
    rows = np.array([N - 1, 0, N // 2])
    y2, S2 = oracle.gemv(q, N, K, xb, rows)
    assert np.array_equal(y2, y[:, rows]) and np.array_equal(S2, S[:, rows])


# ----------------------------------------------------------------------------
# Single-level format (one fp32 absmax per block, no second level)
# ----------------------------------------------------------------------------


def make_sl(packed, absmax, n, bs):
    return oracle.QuantizedSL(np.ascontiguousarray(packed, np.uint8),
                              np.ascontiguousarray(absmax, np.float32), n, bs)


def test_sl_exhaustive_byte_decode(page_table):
    """absmax = 1 everywhere: every packed byte decodes to (NF4[hi], NF4[lo])
    of the page table, the even element from the high nibble."""
    q = make_sl(np.arange(256, dtype=np.uint8), np.ones(8, np.float32), 512, 64)
    v = oracle.dequant_sl_f32(q)
    expect = np.empty(512, np.float32)
    expect[0::2] = page_table[np.arange(256) >> 4]
    expect[1::2] = page_table[np.arange(256) & 15]
    assert np.array_equal(v.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("n,bs", [(4096, 64), (1001, 64), (777, 32), (65, 64), (2, 64), (300, 2),
                                  (513, 128), (5000, 256)])
def test_sl_block_index_closed_form(n, bs):
    """Every code 15 (value +1) and absmax[b] = b + 1/4: element e reads exactly
    e // bs + 1/4; code 0 (-1) gives the negation and code 7 (+0) zeros."""
    nb = (n + bs - 1) // bs
    absmax = (np.arange(nb) + 0.25).astype(np.float32)
    packed = np.full((n + 1) // 2, 0xFF, np.uint8)
    v = oracle.dequant_sl_f32(make_sl(packed, absmax, n, bs)).astype(np.float64)
    expect = np.arange(n) // bs + 0.25
    assert np.array_equal(v, expect)
    v0 = oracle.dequant_sl_f32(make_sl(np.zeros_like(packed), absmax, n, bs)).astype(np.float64)
    assert np.array_equal(v0, -expect)
    v7 = oracle.dequant_sl_f32(make_sl(np.full_like(packed, 0x77), absmax, n, bs))
    assert np.all(v7.view(np.uint32) == 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_sl_dequant_matches_exact_rational(seed, page_table):
    """Exact rationals: the product NF4[idx] * absmax rounded once to fp32
    (subnormal range included); the 16-bit outputs are numpy's (fp16) and
    torch's (bf16) RNE casts of that value."""
    rng = np.random.default_rng(300 + seed)
    n, bs = 1501, 32
    nb = (n + bs - 1) // bs
    packed = rng.integers(0, 256, (n + 1) // 2).astype(np.uint8)
    absmax = (rng.standard_normal(nb) * 2.0 ** rng.integers(-140, 20, nb)).astype(np.float32)
    q = make_sl(packed, absmax, n, bs)
    got = oracle.dequant_sl_f32(q)
    nib = np.empty(2 * packed.size, np.int64)
    nib[0::2] = packed >> 4
    nib[1::2] = packed & 15
    expect = np.array([float(round_fraction(Fraction(float(page_table[nib[e]]))
                                            * Fraction(float(absmax[e // bs]))))
                       for e in range(n)], np.float32)
    # a zero product carries the XOR of the operands' signs (+0 * negative = -0)
    neg = np.signbit(page_table[nib[:n]]) ^ np.signbit(absmax[np.arange(n) // bs])
    expect = np.where(expect == 0, np.where(neg, np.float32(-0.0), np.float32(0.0)), expect)
    assert np.any((expect == 0) & neg)
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
    assert np.array_equal(oracle.dequant_sl(q, oracle.BF16), bf16_bits_torch(expect))
    assert np.array_equal(oracle.dequant_sl(q, oracle.FP16), f16_bits_numpy(expect))


def test_sl_reduces_to_double_quant():
    """With absmax[b] set to the double-quantized tensor's absmax_real (formed
    here with numpy float32 operations: IEEE product, then IEEE sum), the
    single-level dequant equals the double-quantized one bit for bit."""
    q = oracle.quantize(synth.weights(41, 64 * 256 * 2 + 640, outliers=True), 64, 256)
    c2 = q.code2.view(np.float16).astype(np.float32)
    a2 = q.absmax2.view(np.float16).astype(np.float32)
    blk = np.arange(q.nblocks)
    a_real = (c2[q.absmax_q] * a2[blk // q.s2_blocksize]).astype(np.float32) + np.float32(q.offset)
    assert a_real.dtype == np.float32
    sl = make_sl(q.packed, a_real, q.n, q.blocksize)
    for dt in (oracle.BF16, oracle.FP16):
        assert np.array_equal(oracle.dequant_sl(sl, dt), oracle.dequant(q, dt))
    assert np.array_equal(oracle.dequant_sl_f32(sl).view(np.uint32),
                          oracle.dequant_f32(q).view(np.uint32))


def test_sl_sampled_and_ranges_agree():
    q = oracle.quantize_sl(synth.weights(43, 10_007), 64)
    full = oracle.dequant_sl(q, oracle.FP16)
    idx = np.random.default_rng(3).integers(0, q.n, 500)
    assert np.array_equal(oracle.dequant_sl_at(q, idx, oracle.FP16), full[idx])
    assert np.array_equal(oracle.dequant_sl(q, oracle.FP16, 1234, 5678), full[1234:5678])


@pytest.mark.parametrize("n,bs,seed", [(4096, 64, 1), (3001, 64, 2), (255, 32, 3), (1000, 128, 4)])
def test_sl_quantizer_brute_force(n, bs, seed, page_table):
    w = synth.weights(seed, n, outliers=True)
    q = oracle.quantize_sl(w, bs)
    nb = (n + bs - 1) // bs
    wp = np.concatenate([w, np.zeros(nb * bs - n, np.float32)]).reshape(nb, bs)
    absmax = np.abs(wp).max(axis=1)
    assert np.array_equal(q.absmax, absmax)
    r = w / np.repeat(absmax, bs)[:n]
    d = np.abs(r[:, None] - page_table[None, :])
    assert np.array_equal(_nibbles(q), np.argmin(d, axis=1))
    if n % 2:
        assert q.packed[-1] & 15 == 0


def test_sl_quantizer_roundtrip_and_gridpoints():
    """|w - value| <= half the largest NF4 gap times absmax (plus the fp32
    rounding of the product); weights on the grid NF4[j] * A come back as j."""
    w = synth.weights(22, 1 << 15, outliers=True)
    q = oracle.quantize_sl(w)
    t = oracle.nf4_table().astype(np.float64)
    half_gap = np.diff(t).max() / 2
    absmax = np.repeat(q.absmax, 64)[: q.n].astype(np.float64)
    v = oracle.dequant_sl_f32(q).astype(np.float64)
    assert np.all(np.abs(w - v) <= half_gap * absmax * (1 + 2 ** -20) + np.abs(v) * 2 ** -24)
    rng = np.random.default_rng(10)
    A = np.float32(0.01) + rng.random(100, dtype=np.float32)
    j = rng.integers(0, 16, (100, 64))
    j[:, 0] = 0                       # -A in every block: absmax is A
    wg = (oracle.nf4_table()[j] * A[:, None]).astype(np.float32).reshape(-1)
    assert np.array_equal(_nibbles(oracle.quantize_sl(wg)), j.reshape(-1))
    z = oracle.quantize_sl(np.zeros(999, np.float32))
    assert np.all(z.packed[:-1] == 0x77) and z.packed[-1] == 0x70 and np.all(z.absmax == 0)


def test_sl_gemv_one_hot_reproduces_columns():
    N, K = 40, 256
    q = oracle.quantize_sl(synth.weights(5, N * K), 64)
    W = oracle.dequant_sl_f32(q).reshape(N, K)
    for k in (0, 1, 64, 255):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, S = oracle.gemv_sl(q, N, K, synth.to_bf16_bits(x))
        assert np.array_equal(y[0], W[:, k].astype(np.float64))
        assert np.array_equal(S[0], np.abs(W[:, k]).astype(np.float64))


@pytest.mark.parametrize("N,K,B,bs", [(64, 512, 1, 64), (33, 1536, 4, 128), (7, 128, 8, 32)])
def test_sl_gemv_matches_float64_matmul(N, K, B, bs):
    q = oracle.quantize_sl(synth.weights(N + K + 1, N * K), bs)
    W = oracle.dequant_sl_f32(q).reshape(N, K).astype(np.float64)
    xb = synth.activations(8, B, K)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    y, S = oracle.gemv_sl(q, N, K, xb)
    assert np.allclose(y, xf @ W.T, rtol=1e-12, atol=1e-12 * np.abs(xf) @ np.abs(W).T)
    assert np.allclose(S, np.abs(xf) @ np.abs(W).T, rtol=1e-12)
    rows = np.array([N - 1, 0])
    y2, S2 = oracle.gemv_sl(q, N, K, xb, rows)
    assert np.array_equal(y2, y[:, rows]) and np.array_equal(S2, S[:, rows])


# ----------------------------------------------------------------------------
# INT4 asymmetric group format (handbook page: "量化公式", "W4A16：在寄存器里反量化")
# ----------------------------------------------------------------------------

F16 = np.float16


def make_i4(packed, scales, zeros, n, G):
    return oracle.QuantizedInt4(np.ascontiguousarray(packed, np.uint8),
                                np.ascontiguousarray(np.asarray(scales, F16).view(np.uint16)),
                                np.ascontiguousarray(np.asarray(zeros, F16).view(np.uint16)), n, G)


def test_int4_word_layout_is_low_nibble_first():
    """The page stores 8 consecutive weights per 32-bit word with the first
    one in the low 4 bits: element 8 i + j is (word_i >> 4 j) & 15."""
    rng = np.random.default_rng(50)
    words = rng.integers(0, 2 ** 32, 64, dtype=np.uint64).astype(np.uint32)
    packed = words.view(np.uint8)             # little-endian bytes of the words
    n = 8 * words.size
    q = make_i4(packed, np.ones(n // 128), np.zeros(n // 128), n, 128)
    v = oracle.int4_dequant_f32(q)
    expect = ((words[:, None] >> (4 * np.arange(8, dtype=np.uint32))[None, :]) & 15).reshape(-1)
    assert np.array_equal(v, expect.astype(np.float32))


def test_int4_exhaustive_byte_decode():
    q = make_i4(np.arange(256, dtype=np.uint8), [1.0] * 4, [0.0] * 4, 512, 128)
    v = oracle.int4_dequant_f32(q)
    assert np.array_equal(v[0::2], (np.arange(256) & 15).astype(np.float32))
    assert np.array_equal(v[1::2], (np.arange(256) >> 4).astype(np.float32))


@pytest.mark.parametrize("n,G", [(4096, 128), (1000, 128), (777 * 2, 32), (64, 64), (300, 2)])
def test_int4_dequant_closed_form(n, G):
    """Power-of-two scales and integer zero points: every value is the exact
    (q - z) * s."""
    ng = -(-n // G)
    rng = np.random.default_rng(n + G)
    s = 2.0 ** (np.arange(ng) % 12 - 6)
    z = np.arange(ng) % 17 - 1                    # includes -1 and 15
    packed = rng.integers(0, 256, (n + 1) // 2).astype(np.uint8)
    v = oracle.int4_dequant_f32(make_i4(packed, s, z, n, G)).astype(np.float64)
    e = np.arange(n)
    qv = np.where(e % 2 == 0, packed[e // 2] & 15, packed[e // 2] >> 4).astype(np.float64)
    assert np.array_equal(v, (qv - z[e // G]) * s[e // G])


@pytest.mark.parametrize("seed", [0, 1])
def test_int4_dequant_matches_exact_rational(seed):
    """Exact rationals with arbitrary fp16 scales (subnormals included) and
    non-integer fp16 zero points: q - z is exact in fp32, the product is
    rounded once; the 16-bit outputs are numpy / torch RNE casts of it."""
    rng = np.random.default_rng(400 + seed)
    n, G = 1024, 32
    ng = n // G
    packed = rng.integers(0, 256, n // 2).astype(np.uint8)
    s = (rng.standard_normal(ng) * 2.0 ** rng.integers(-26, 4, ng)).astype(F16)
    z = (rng.standard_normal(ng) * 8).astype(F16)
    q = make_i4(packed, s, z, n, G)
    got = oracle.int4_dequant_f32(q)
    e = np.arange(n)
    qv = np.where(e % 2 == 0, packed[e // 2] & 15, packed[e // 2] >> 4)
    expect = np.array([float(round_fraction((Fraction(int(qv[i])) - Fraction(float(z[i // G])))
                                            * Fraction(float(s[i // G])))) for i in range(n)],
                      np.float32)
    neg = np.signbit(s[e // G].astype(np.float32)) ^ ((qv - z[e // G].astype(np.float64)) < 0)
    expect = np.where(expect == 0, np.where(neg, np.float32(-0.0), np.float32(0.0)), expect)
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
    assert np.array_equal(oracle.int4_dequant(q, oracle.BF16), bf16_bits_torch(expect))
    assert np.array_equal(oracle.int4_dequant(q, oracle.FP16), f16_bits_numpy(expect))


def test_int4_quantizer_grid_round_trip():
    """Groups built on the grid (q - z) s with s a power of two, z an integer
    in 0..15 and both q = 0 and q = 15 present: min = -z s and max = (15 - z) s,
    so the quantizer recovers s, z and every code exactly."""
    rng = np.random.default_rng(11)
    G, ng = 128, 64
    s = 2.0 ** rng.integers(-12, -2, ng)
    z = rng.integers(0, 16, ng)
    q = rng.integers(0, 16, (ng, G))
    q[:, 0], q[:, 1] = 0, 15
    w = ((q - z[:, None]) * s[:, None]).astype(np.float32).reshape(-1)
    got = oracle.int4_quantize(w, G)
    assert np.array_equal(got.scales.view(F16).astype(np.float64), s)
    assert np.array_equal(got.zeros.view(F16).astype(np.float64), z.astype(np.float64))
    codes = np.empty(w.size, np.int64)
    codes[0::2] = got.packed & 15
    codes[1::2] = got.packed >> 4
    assert np.array_equal(codes, q.reshape(-1))


def test_int4_quantizer_bounds():
    """Random weights: s is the fp16 rounding of (max - min) / 15, z is within
    1/2 of -min / s, codes are in range, and each weight is within one step s
    of its value (half a step plus the fp16 rounding of s times 15 at most)."""
    G = 128
    w = synth.weights(12, 64 * G, outliers=True)
    q = oracle.int4_quantize(w, G)
    wg = w.reshape(-1, G).astype(np.float64)
    s = q.scales.view(F16).astype(np.float64)
    z = q.zeros.view(F16).astype(np.float64)
    span = wg.max(axis=1) - wg.min(axis=1)
    assert np.all(np.abs(s - span / 15) <= 2.0 ** -11 * span / 15 + 1e-12)
    assert np.all(np.abs(-wg.min(axis=1) / s - z) <= 0.5 + 1e-6)
    v = oracle.int4_dequant_f32(q).astype(np.float64).reshape(-1, G)
    assert np.all(np.abs(wg - v) <= s[:, None] * (0.5 + 15 * 2.0 ** -11) + 1e-9)


def test_int4_quantizer_constant_and_zero_groups():
    w = np.concatenate([np.zeros(128), np.full(128, 0.3), np.full(128, -2.7)]).astype(np.float32)
    q = oracle.int4_quantize(w, 128)
    assert np.all(q.scales.view(F16) == 1.0)          # a zero span takes scale 1
    v = oracle.int4_dequant_f32(q).reshape(3, 128)
    assert np.all(v[0] == 0.0)
    assert np.all(np.abs(v[1:] - w.reshape(3, 128)[1:]) <= 0.5)


def test_int4_quantizer_halves_round_away_from_zero():
    """Exact halves.  One group of 16 with min -6.5 and max 8.5: the span is
    15, so s = 1 exactly and -min / s = 6.5 rounds away from zero to z = 7
    (round-half-even would give 6).  The formula rounds w / s first and then
    adds z: w = -0.5 gives round(-0.5) + 7 = 6, where rounding w / s + z = 6.5
    as one value would give 7; w = 0.5 gives 8, w = 2.5 gives 10 (half-even:
    8 with z = 6), w = 1.5 gives 9, -6.5 gives 0 and 8.5 gives 16, clamped to
    15."""
    w = np.zeros(16, np.float32)
    w[:8] = [-6.5, 8.5, -0.5, 0.5, 2.5, 1.5, -2.5, 0.0]
    q = oracle.int4_quantize(w, 16)
    assert q.scales.view(F16)[0] == 1.0
    assert q.zeros.view(F16)[0] == 7.0
    codes = np.empty(16, np.int64)
    codes[0::2] = q.packed & 15
    codes[1::2] = q.packed >> 4
    assert codes[:8].tolist() == [0, 15, 6, 8, 10, 9, 4, 7]


def test_int4_gemv_one_hot_and_magnitudes():
    N, K, G = 24, 512, 128
    q = oracle.int4_quantize(synth.weights(13, N * K), G)
    W = oracle.int4_dequant_f32(q).reshape(N, K)
    for k in (0, 1, 127, 128, 511):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, S, M = oracle.int4_gemv(q, N, K, synth.to_bf16_bits(x))
        assert np.array_equal(y[0], W[:, k].astype(np.float64))
        assert np.array_equal(S[0], np.abs(W[:, k]).astype(np.float64))
        codes = np.empty(N * K, np.int64)
        codes[0::2] = q.packed & 15
        codes[1::2] = q.packed >> 4
        grp = (np.arange(N) * K + k) // G
        s = q.scales.view(F16).astype(np.float64)[grp]
        z = q.zeros.view(F16).astype(np.float64)[grp]
        assert np.allclose(M[0], (codes.reshape(N, K)[:, k] + np.abs(z)) * np.abs(s), rtol=1e-15)


@pytest.mark.parametrize("N,K,B,G", [(64, 512, 1, 128), (33, 1536, 4, 128), (7, 256, 8, 32)])
def test_int4_gemv_matches_float64_matmul(N, K, B, G):
    q = oracle.int4_quantize(synth.weights(N + K + 2, N * K), G)
    W = oracle.int4_dequant_f32(q).reshape(N, K).astype(np.float64)
    xb = synth.activations(9, B, K)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    y, S, M = oracle.int4_gemv(q, N, K, xb)
    assert np.allclose(y, xf @ W.T, rtol=1e-12, atol=1e-12 * np.abs(xf) @ np.abs(W).T)
    assert np.allclose(S, np.abs(xf) @ np.abs(W).T, rtol=1e-12)
    assert np.all(M >= S * (1 - 1e-12))
    rows = np.array([N - 1, 0])
    y2, S2, M2 = oracle.int4_gemv(q, N, K, xb, rows)
    assert np.array_equal(y2, y[:, rows]) and np.array_equal(M2, M[:, rows])
