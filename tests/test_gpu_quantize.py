"""GPU quantizer parity: nf4_quantize (through the C ABI) against the oracle
quantizer on the same fp32 weights.  Every output -- packed codes, absmax_q,
absmax2 and the offset -- must be bit-identical: each decision is an exact or
correctly rounded fp32 operation on both sides, and the offset is one fp64
sum in block-index order on both."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu

CASES = [
    # n, blocksize, s2, outliers
    (1 << 20, 64, 256, False), (4096 * 4096, 64, 256, True), (2047 * 4096, 64, 256, False),
    (1, 64, 256, False), (2, 64, 256, False), (63, 64, 256, True), (64 * 1024 * 3 + 7, 64, 256, True),
    (100_001, 32, 4, True), (70_000, 128, 1, False), (5000, 8, 2, True), (3001, 1, 8, False),
    (1024 * 64 * 5 + 1, 64, 256, False),
]


def quantize_on_gpu(w, bs, s2):
    wt = torch.from_numpy(w).to(G.dev())
    print(f"[quantize] n={w.size} bs={bs} s2={s2}", flush=True)
    t = nf4.nf4_quantize(wt, bs, s2)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("n,bs,s2,outliers", CASES)
def test_quantize_matches_oracle(n, bs, s2, outliers):
    w = synth.weights(n + 3 * bs + s2, n, outliers=outliers)
    ref = oracle.quantize(w, bs, s2)
    got = quantize_on_gpu(w, bs, s2)
    assert np.float32(got.offset).view(np.uint32) == np.float32(ref.offset).view(np.uint32)
    assert np.array_equal(G.bits16(got.absmax2), ref.absmax2)
    assert np.array_equal(got.absmax_q.cpu().numpy(), ref.absmax_q)
    assert np.array_equal(got.packed.cpu().numpy(), ref.packed)


@pytest.mark.parametrize("case", ["big_first", "tiny_first"])
def test_quantize_offset_sums_in_block_order(case):
    """Block absmax values for which the order of the fp64 sum shows in the
    fp32 offset (the cases of the oracle pin
    test_quantizer_offset_is_the_index_order_fp64_mean): the device must
    reach the same bits, 2^-11 and 2^-11 + 2^-34."""
    a = np.zeros(2048, np.float32)
    if case == "big_first":
        a[0], a[1], a[1024:1027] = 1.0, 2.0 ** -24, 2.0 ** -54
        expect = np.float32(2.0 ** -11)
    else:
        a[0:3], a[3], a[4] = 2.0 ** -54, 1.0, 2.0 ** -24
        expect = np.float32(2.0 ** -11 + 2.0 ** -34)
    w = np.zeros((2048, 64), np.float32)
    w[:, 0] = a
    w = w.reshape(-1)
    ref = oracle.quantize(w)
    got = quantize_on_gpu(w, 64, 256)
    assert np.float32(ref.offset) == expect
    assert np.float32(got.offset).view(np.uint32) == expect.view(np.uint32)
    assert np.array_equal(G.bits16(got.absmax2), ref.absmax2)
    assert np.array_equal(got.absmax_q.cpu().numpy(), ref.absmax_q)


def test_quantize_zero_blocks_and_exact_grid_points():
    rng = np.random.default_rng(3)
    t = oracle.nf4_table()
    nb = 512
    j = rng.integers(0, 16, (nb, 64))
    j[:, 0] = 15
    A = (0.01 + rng.random(nb)).astype(np.float32)
    w = (t[j] * A[:, None]).astype(np.float32)
    w[::7] = 0.0                       # whole zero blocks
    w = w.reshape(-1)
    ref = oracle.quantize(w)
    got = quantize_on_gpu(w, 64, 256)
    assert np.array_equal(got.packed.cpu().numpy(), ref.packed)
    assert np.array_equal(got.absmax_q.cpu().numpy(), ref.absmax_q)


def test_quantize_dequant_round_trip_on_gpu():
    """GPU quantize then GPU dequant equals the oracle's dequant of the
    oracle's encoding."""
    w = synth.weights(44, 1 << 18, outliers=True)
    got = quantize_on_gpu(w, 64, 256)
    out = got.dequant()
    torch.cuda.synchronize()
    assert np.array_equal(G.bits16(out), oracle.dequant(oracle.quantize(w)))


def test_quantize_is_deterministic():
    w = synth.weights(45, 1 << 20)
    a = quantize_on_gpu(w, 64, 256)
    b = quantize_on_gpu(w, 64, 256)
    assert a.offset == b.offset
    assert torch.equal(a.packed, b.packed) and torch.equal(a.absmax_q, b.absmax_q)


# ---------------------------------------------------------------------------
# single-level format
# ---------------------------------------------------------------------------

SL_CASES = [(1 << 20, 64, False), (4096 * 4096, 64, True), (1, 64, False), (63, 64, True),
            (100_001, 32, True), (70_000, 128, False), (5000, 8, True), (3001, 1, False)]


@pytest.mark.parametrize("n,bs,outliers", SL_CASES)
def test_quantize_absmax32_matches_oracle(n, bs, outliers):
    w = synth.weights(n + 5 * bs, n, outliers=outliers)
    ref = oracle.quantize_sl(w, bs)
    print(f"[quantize_absmax32] n={n} bs={bs}", flush=True)
    got = nf4.nf4_quantize_absmax32(torch.from_numpy(w).to(G.dev()), bs)
    torch.cuda.synchronize()
    assert np.array_equal(got.absmax.cpu().numpy().view(np.uint32), ref.absmax.view(np.uint32))
    assert np.array_equal(got.packed.cpu().numpy(), ref.packed)


def test_quantize_absmax32_round_trip_on_gpu():
    """GPU single-level encode, then GPU dequant and GEMV, against the oracle
    on its own encoding of the same weights."""
    N, K = 512, 4096
    w = synth.weights(46, N * K, outliers=True)
    got = nf4.nf4_quantize_absmax32(torch.from_numpy(w).to(G.dev()), 64)
    out = got.dequant()
    xb = synth.activations(47, 2, K)
    y = got.gemv(N, K, G.x_to_device(xb))
    torch.cuda.synchronize()
    ref = oracle.quantize_sl(w, 64)
    assert np.array_equal(G.bits16(out), oracle.dequant_sl(ref))
    yr, S = oracle.gemv_sl(ref, N, K, xb)
    ok, worst = G.gemv_within_tolerance(G.bf16_to_f64(G.bits16(y)), yr, S)
    assert ok, worst
