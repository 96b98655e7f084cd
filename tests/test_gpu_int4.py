"""GPU parity for the INT4 asymmetric group format (include/int4.h) through
the C ABI against the oracle on the same seeded inputs.

Dequant and the GPU encoder must be bit-exact.  GEMV outputs must be the bf16
rounding (nearest even) of a real within 2^-14 M of the fp64 oracle value,
M = sum_k (|q| + |z|) |s| |x_k|: the main kernels apply each group's zero point
once per lane piece (s (sum q x - z sum x)), so their rounding error scales
with those sums rather than with sum |w x|."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu

DT = {oracle.BF16: torch.bfloat16, oracle.FP16: torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nf4.load()


def to_dev(q):
    return G.u8(q.packed), G.h16(q.scales), G.h16(q.zeros)


def run_dequant(q, out_dtype=oracle.BF16, offset_elems=0, packed_offset=0):
    packed, scales, zeros = to_dev(q)
    if packed_offset:
        buf = torch.zeros(q.packed.size + packed_offset, dtype=torch.uint8, device=G.dev())
        buf[packed_offset:] = packed
        packed = buf[packed_offset:]
    base, out = G.guarded(q.n, DT[out_dtype], offset_elems)
    print(f"[int4_dequant] n={q.n} G={q.group} dtype={out_dtype} out_off={offset_elems} "
          f"packed_off={packed_offset}", flush=True)
    nf4.int4_dequant(packed, scales, zeros, q.n, q.group, out=out)
    torch.cuda.synchronize()
    assert G.guards_intact(base, q.n, offset_elems), "write outside the output buffer"
    return G.bits16(out)


def assert_bits_equal(got, ref):
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError(f"{bad.size} of {ref.size} elements differ; first at {bad[:8]}: "
                             f"gpu {got[bad[:8]]} oracle {ref[bad[:8]]}")


# ---------------------------------------------------------------------------
# dequant and encoder
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_int4_dequant_4096x4096_outliers(dtype):
    cfg = synth.DEQUANT_4K
    q = oracle.int4_quantize(synth.weights(cfg.seed, cfg.n, outliers=True), 128)
    assert_bits_equal(run_dequant(q, dtype), oracle.int4_dequant(q, dtype))


INT4_EDGE = [
    (2, 128), (8, 128), (9, 128), (63, 128), (65, 128), (12345, 128), (2047 * 4096, 128),
    (100_003, 128), (4096, 8), (4099, 16), (5000, 32), (5000, 64), (5000, 256), (3001, 4),
    (3001, 2), (70_000, 1 << 14),
    (1_048_575, 128), (1_500_001, 128), (2_097_147, 128), (2_100_003, 8),
]


@pytest.mark.parametrize("n,g", INT4_EDGE)
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_int4_dequant_edge_shapes(n, g, dtype):
    q = oracle.int4_quantize(synth.weights(n + g + 1, n, outliers=True), g)
    assert_bits_equal(run_dequant(q, dtype), oracle.int4_dequant(q, dtype))


@pytest.mark.parametrize("offset_elems,packed_offset", [(1, 0), (0, 1), (3, 2)])
def test_int4_dequant_unaligned_buffers(offset_elems, packed_offset):
    q = oracle.int4_quantize(synth.weights(33, 50_001), 128)
    assert_bits_equal(run_dequant(q, oracle.BF16, offset_elems, packed_offset),
                      oracle.int4_dequant(q, oracle.BF16))


@pytest.mark.parametrize("g", [128, 4])
def test_int4_dequant_special_values(g):
    """Every byte value with fp16 scales of any sign and size (subnormals,
    values whose products overflow fp16) and non-integer zero points."""
    rng = np.random.default_rng(g)
    n = 512 * 40
    ng = n // g
    packed = np.tile(np.arange(256, dtype=np.uint8), n // 512)
    # finite fp16 scales only (|s| <= 65504): the draw is clipped before the cast
    s = np.clip(rng.standard_normal(ng) * 2.0 ** rng.integers(-24, 16, ng), -65504.0,
                65504.0).astype(np.float16)
    assert np.all(np.isfinite(s))
    z = (rng.standard_normal(ng) * 20).astype(np.float16)
    s[:4] = [0.0, -0.0, 6e-8, 65504.0]
    q = oracle.QuantizedInt4(packed, s.view(np.uint16), z.view(np.uint16), n, g)
    for dtype in (oracle.BF16, oracle.FP16):
        with np.errstate(over="ignore"):
            assert_bits_equal(run_dequant(q, dtype), oracle.int4_dequant(q, dtype))


@pytest.mark.parametrize("n,g,outliers", [(1 << 20, 128, False), (4096 * 4096, 128, True),
                                          (1, 128, False), (63, 128, True), (100_001, 32, True),
                                          (70_000, 256, False), (5000, 8, True), (3001, 2, False)])
def test_int4_quantize_matches_oracle(n, g, outliers):
    w = synth.weights(n + 7 * g, n, outliers=outliers)
    ref = oracle.int4_quantize(w, g)
    print(f"[int4_quantize] n={n} G={g}", flush=True)
    got = nf4.int4_quantize(torch.from_numpy(w).to(G.dev()), g)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits16(got.scales), ref.scales)
    assert np.array_equal(G.bits16(got.zeros), ref.zeros)
    assert np.array_equal(got.packed.cpu().numpy(), ref.packed)


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------


def run_gemv(q, N, K, xbits, x_offset=0):
    B = xbits.shape[0]
    packed, scales, zeros = to_dev(q)
    x = G.x_to_device(xbits)
    if x_offset:
        buf = torch.zeros(B * K + x_offset, dtype=torch.bfloat16, device=G.dev())
        buf[x_offset:] = x.reshape(-1)
        x = buf[x_offset:].view(B, K)
    base, yv = G.guarded(B * N, torch.bfloat16)
    print(f"[int4_gemv] N={N} K={K} B={B} G={q.group} x_off={x_offset}", flush=True)
    nf4.int4_gemv(packed, scales, zeros, N, K, x, q.group, y=yv.view(B, N))
    torch.cuda.synchronize()
    assert G.guards_intact(base, B * N), "write outside y"
    return G.bf16_to_f64(G.bits16(yv)).reshape(B, N)


def check_gemv(q, N, K, xbits, x_offset=0):
    y = run_gemv(q, N, K, xbits, x_offset)
    yr, _, M = oracle.int4_gemv(q, N, K, xbits)
    ok, worst = G.gemv_within_tolerance(y, yr, M)
    assert ok, f"INT4 GEMV N={N} K={K} B={xbits.shape[0]}: worst error/bound = {worst:.3g}"


@pytest.mark.parametrize("g", synth.QWEN_GEMVS, ids=lambda g: g.name)
def test_int4_gemv_qwen_batch1(g):
    q = oracle.int4_quantize(synth.weights(g.seed, g.N * g.K), 128)
    check_gemv(q, g.N, g.K, synth.activations(synth.QWEN_X_SEED, 1, g.K))


@pytest.mark.parametrize("batch", synth.LLAMA_BATCHES)
@pytest.mark.parametrize("g", synth.LLAMA_GEMVS, ids=lambda g: g.name)
def test_int4_gemv_llama(g, batch):
    q = oracle.int4_quantize(synth.weights(g.seed, g.N * g.K), 128)
    check_gemv(q, g.N, g.K, synth.activations(synth.llama_x_seed(batch), batch, g.K))


INT4_GEMV_EDGE = [
    # N, K, G
    (1, 128, 128), (3, 256, 128), (5, 2048, 128), (7, 2080, 32), (33, 32, 32), (17, 96, 32),
    (9, 16384, 128), (3, 16416, 32), (11, 1000, 8), (13, 2, 2), (6, 130, 2), (300, 1536, 128),
    (257, 1536, 16), (64, 4096, 4096), (1376, 4096, 128), (4096, 1376, 32), (100, 8192, 256),
    (50, 12288, 128), (4096, 4096, 64), (40, 12352, 64), (21, 2112, 64), (19, 4160, 64),
]


@pytest.mark.parametrize("N,K,g", INT4_GEMV_EDGE)
@pytest.mark.parametrize("batch", [1, 2, 3, 8])
def test_int4_gemv_edge_shapes(N, K, g, batch):
    q = oracle.int4_quantize(synth.weights(N * 3 + K, N * K, outliers=True), g)
    check_gemv(q, N, K, synth.activations(N + K + batch + 1, batch, K))


@pytest.mark.parametrize("batch", [1, 5, 8])
def test_int4_gemv_unaligned_x(batch):
    N, K = 40, 4096
    q = oracle.int4_quantize(synth.weights(25, N * K), 128)
    check_gemv(q, N, K, synth.activations(26, batch, K), x_offset=1)


@pytest.mark.parametrize("N,batch", [(256, 1), (256, 2), (256, 4), (256, 8), (8192, 1)])
def test_int4_gemv_one_hot_is_exact(N, batch):
    """x = e_k: the codes are exact in bf16 and s (q - z) is rounded once, as
    the oracle rounds (q - z) s, so y[r] is exactly the bf16 of W[r][k]."""
    K = 4096
    q = oracle.int4_quantize(synth.weights(28, N * K), 128)
    W = oracle.int4_dequant_f32(q).reshape(N, K)
    ks = [0, 127, 128, 2047, 4095, 1000, 3000, 17][:batch]
    x = np.zeros((batch, K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    y = run_gemv(q, N, K, synth.to_bf16_bits(x))
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], G.bf16_to_f64(oracle.bf16_from_f32(W[:, k]))), (b, k)


def test_int4_gemv_empty_k_gives_zeros():
    N, B = 100, 2
    y = torch.full((B, N), 7.0, dtype=torch.bfloat16, device=G.dev())
    z8 = torch.zeros(1, dtype=torch.uint8, device=G.dev())
    z16 = torch.zeros(1, dtype=torch.int16, device=G.dev())
    nf4.int4_gemv(z8, z16, z16, N, 0, torch.zeros((B, 0), dtype=torch.bfloat16, device=G.dev()),
                  128, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_int4_gemv_round_trip_on_gpu():
    """GPU encode, then GPU dequant and GEMV, against the oracle on its own
    encoding of the same weights."""
    N, K = 512, 4096
    w = synth.weights(29, N * K, outliers=True)
    t = nf4.int4_quantize(torch.from_numpy(w).to(G.dev()), 128)
    out = t.dequant()
    xb = synth.activations(30, 3, K)
    y = t.gemv(N, K, G.x_to_device(xb))
    torch.cuda.synchronize()
    ref = oracle.int4_quantize(w, 128)
    assert np.array_equal(G.bits16(out), oracle.int4_dequant(ref))
    yr, _, M = oracle.int4_gemv(ref, N, K, xb)
    ok, worst = G.gemv_within_tolerance(G.bf16_to_f64(G.bits16(y)), yr, M)
    assert ok, worst


@pytest.mark.parametrize("batch", [1, 4])
def test_int4_gemv_past_2g_weights_sampled_rows(batch):
    """N * K just above 2^31 (the kernel past the streaming kernels' 32-bit
    offsets): random codes, scales and zero points drawn on the device; 64
    sampled rows checked against the oracle (K % G == 0, so a row's groups
    are its own)."""
    K, g = 4096, 128
    N = (1 << 31) // K + 64
    n = N * K
    gen = torch.Generator(device=G.dev())
    gen.manual_seed(900 + batch)
    packed = torch.randint(0, 256, (n // 2,), dtype=torch.uint8, device=G.dev(), generator=gen)
    ng = n // g
    scales = (torch.rand(ng, device=G.dev(), generator=gen) * 0.01 + 1e-3).to(torch.float16)
    zeros = torch.randint(0, 16, (ng,), device=G.dev(), generator=gen).to(torch.float16)
    xbits = synth.activations(910 + batch, batch, K)
    y = torch.empty((batch, N), dtype=torch.bfloat16, device=G.dev())
    print(f"[int4_gemv_past_2g] N={N} K={K} B={batch}", flush=True)
    nf4.int4_gemv(packed, scales, zeros, N, K, G.x_to_device(xbits), g, y=y)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(920 + batch).choice(N, 64, replace=False))
    rt = torch.from_numpy(rows).to(G.dev())
    sub = oracle.QuantizedInt4(packed.view(N, K // 2)[rt].cpu().numpy().reshape(-1),
                               G.bits16(scales.view(N, K // g)[rt]).reshape(-1),
                               G.bits16(zeros.view(N, K // g)[rt]).reshape(-1), rows.size * K, g)
    yr, _, M = oracle.int4_gemv(sub, rows.size, K, xbits)
    got = G.bf16_to_f64(G.bits16(y[:, rt]))
    ok, worst = G.gemv_within_tolerance(got, yr, M)
    assert ok, f"worst error/bound = {worst:.3g}"
    del packed
    torch.cuda.empty_cache()
