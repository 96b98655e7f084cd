"""GPU parity for the single-level format (one fp32 absmax per block, no
second level): nf4_dequant_absmax32 and nf4_gemv_absmax32 through the C ABI
against the oracle on the same seeded inputs.  Dequant must be bit-exact
(signed zeros included); GEMV outputs must meet the rule of tests/_gpu.py.
Also the GEMV of matrices with N*K >= 2^31 elements in both formats (the
kernel past the 32-bit offsets of the streaming kernels), checked on sampled
rows."""
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


def f32dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(G.dev())


def run_dequant_sl(q, out_dtype=oracle.BF16, offset_elems=0, packed_offset=0):
    packed = G.u8(q.packed)
    if packed_offset:
        buf = torch.zeros(q.packed.size + packed_offset, dtype=torch.uint8, device=G.dev())
        buf[packed_offset:] = packed
        packed = buf[packed_offset:]
    base, out = G.guarded(q.n, DT[out_dtype], offset_elems)
    print(f"[dequant_absmax32] n={q.n} bs={q.blocksize} dtype={out_dtype} "
          f"out_off={offset_elems} packed_off={packed_offset}", flush=True)
    nf4.nf4_dequant_absmax32(packed, f32dev(q.absmax), q.n, q.blocksize, out=out)
    torch.cuda.synchronize()
    assert G.guards_intact(base, q.n, offset_elems), "write outside the output buffer"
    return G.bits16(out)


def assert_bits_equal(got, ref):
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError(f"{bad.size} of {ref.size} elements differ; first at {bad[:8]}: "
                             f"gpu {got[bad[:8]]} oracle {ref[bad[:8]]}")


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------


def test_dequant_absmax32_1024x1024():
    cfg = synth.DEQUANT_1K
    q = oracle.quantize_sl(synth.weights(cfg.seed, cfg.n), 64)
    assert_bits_equal(run_dequant_sl(q), oracle.dequant_sl(q))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_dequant_absmax32_4096x4096_outliers(dtype):
    cfg = synth.DEQUANT_4K
    q = oracle.quantize_sl(synth.weights(cfg.seed, cfg.n, outliers=True), 64)
    assert_bits_equal(run_dequant_sl(q, dtype), oracle.dequant_sl(q, dtype))


SL_EDGE = [
    (1, 64), (2, 64), (7, 64), (8, 64), (9, 64), (63, 64), (65, 64), (12345, 64),
    (2047 * 4096, 64), (100_003, 64), (4096, 8), (4099, 16), (5000, 32), (5000, 128),
    (3001, 4), (3001, 2), (777, 1), (70_000, 1 << 14),
    # tile-size boundaries of the vector path (1, 2, 4 steps per lane on 256
    # CUs) with ragged tails; blocksize 8 fills the scale table
    (1_048_575, 64), (1_500_001, 64), (2_097_147, 64), (2_100_003, 8),
]


@pytest.mark.parametrize("n,bs", SL_EDGE)
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_dequant_absmax32_edge_shapes(n, bs, dtype):
    q = oracle.quantize_sl(synth.weights(n + bs, n, outliers=True), bs)
    assert_bits_equal(run_dequant_sl(q, dtype), oracle.dequant_sl(q, dtype))


@pytest.mark.parametrize("offset_elems,packed_offset", [(1, 0), (0, 1), (3, 2)])
def test_dequant_absmax32_unaligned_buffers(offset_elems, packed_offset):
    q = oracle.quantize_sl(synth.weights(32, 50_001), 64)
    got = run_dequant_sl(q, oracle.BF16, offset_elems, packed_offset)
    assert_bits_equal(got, oracle.dequant_sl(q, oracle.BF16))


@pytest.mark.parametrize("bs", [64, 4])
def test_dequant_absmax32_special_values(bs):
    """Every byte value, with scales that are +-0, negative, subnormal, tiny,
    and large enough to overflow fp16 (to +-inf) or to round to bf16 ties."""
    rng = np.random.default_rng(bs)
    n = 256 * 2 * 40
    nb = n // bs
    packed = np.tile(np.arange(256, dtype=np.uint8), n // 512)
    absmax = (rng.standard_normal(nb) * 2.0 ** rng.integers(-149, 24, nb)).astype(np.float32)
    absmax[:8] = [0.0, -0.0, 1e-45, -1e-45, 3e38, -3e38, 65520.0, 1.0 + 2.0 ** -8]
    q = oracle.QuantizedSL(packed, absmax, n, bs)
    for dtype in (oracle.BF16, oracle.FP16):
        assert_bits_equal(run_dequant_sl(q, dtype), oracle.dequant_sl(q, dtype))


def test_dequant_absmax32_8192x28672():
    cfg = synth.DEQUANT_BIG
    q = oracle.quantize_sl(synth.weights(cfg.seed, cfg.n), 64)
    assert_bits_equal(run_dequant_sl(q, oracle.BF16), oracle.dequant_sl(q, oracle.BF16))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------


def run_gemv_sl(q, N, K, xbits, x_offset=0):
    B = xbits.shape[0]
    x = G.x_to_device(xbits)
    if x_offset:
        buf = torch.zeros(B * K + x_offset, dtype=torch.bfloat16, device=G.dev())
        buf[x_offset:] = x.reshape(-1)
        x = buf[x_offset:].view(B, K)
    base, yv = G.guarded(B * N, torch.bfloat16)
    print(f"[gemv_absmax32] N={N} K={K} B={B} bs={q.blocksize} x_off={x_offset}", flush=True)
    nf4.nf4_gemv_absmax32(G.u8(q.packed), f32dev(q.absmax), N, K, x, q.blocksize,
                          y=yv.view(B, N))
    torch.cuda.synchronize()
    assert G.guards_intact(base, B * N), "write outside y"
    return G.bf16_to_f64(G.bits16(yv)).reshape(B, N)


def check_gemv_sl(q, N, K, xbits, x_offset=0):
    y = run_gemv_sl(q, N, K, xbits, x_offset)
    yr, S = oracle.gemv_sl(q, N, K, xbits)
    ok, worst = G.gemv_within_tolerance(y, yr, S)
    assert ok, f"GEMV N={N} K={K} B={xbits.shape[0]}: worst error/bound = {worst:.3g}"


@pytest.mark.parametrize("g", synth.QWEN_GEMVS, ids=lambda g: g.name)
def test_gemv_absmax32_qwen_batch1(g):
    q = oracle.quantize_sl(synth.weights(g.seed, g.N * g.K), 64)
    check_gemv_sl(q, g.N, g.K, synth.activations(synth.QWEN_X_SEED, 1, g.K))


@pytest.mark.parametrize("batch", synth.LLAMA_BATCHES)
@pytest.mark.parametrize("g", synth.LLAMA_GEMVS, ids=lambda g: g.name)
def test_gemv_absmax32_llama(g, batch):
    q = oracle.quantize_sl(synth.weights(g.seed, g.N * g.K), 64)
    check_gemv_sl(q, g.N, g.K, synth.activations(synth.llama_x_seed(batch), batch, g.K))


SL_GEMV_EDGE = [
    # N, K, bs
    (1, 64, 64), (3, 64, 64), (5, 2048, 64), (7, 2080, 64), (33, 32, 32), (17, 96, 32),
    (9, 16384, 64), (3, 16416, 64), (11, 1000, 64), (13, 2, 64), (6, 130, 2),
    (300, 1536, 128), (257, 1536, 16), (64, 4096, 1 << 12), (1376, 4096, 64),
    (4096, 1376, 64), (100, 8192, 64), (50, 12288, 64), (40, 12352, 64), (21, 2112, 64),
    (19, 4160, 128),
]


@pytest.mark.parametrize("N,K,bs", SL_GEMV_EDGE)
@pytest.mark.parametrize("batch", [1, 2, 3, 8])
def test_gemv_absmax32_edge_shapes(N, K, bs, batch):
    q = oracle.quantize_sl(synth.weights(N * 5 + K, N * K, outliers=True), bs)
    check_gemv_sl(q, N, K, synth.activations(N + K + batch, batch, K))


@pytest.mark.parametrize("batch", [1, 5, 8])
def test_gemv_absmax32_unaligned_x(batch):
    N, K = 40, 4096
    q = oracle.quantize_sl(synth.weights(15, N * K), 64)
    check_gemv_sl(q, N, K, synth.activations(16, batch, K), x_offset=1)


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv_absmax32_one_hot_picks_the_column(batch):
    """x = e_k: y[r] is the single product W[r][k] up to the decode table's
    2^-16 (G.one_hot_ok)."""
    N, K = 256, 4096
    q = oracle.quantize_sl(synth.weights(18, N * K), 64)
    W = oracle.dequant_sl_f32(q).reshape(N, K)
    ks = [0, 63, 64, 2047, 4095, 1000, 3000, 17][:batch]
    x = np.zeros((batch, K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    y = run_gemv_sl(q, N, K, synth.to_bf16_bits(x))
    for b, k in enumerate(ks):
        assert G.one_hot_ok(y[b], W[:, k]), (b, k)


def test_gemv_absmax32_empty_k_gives_zeros():
    N, B = 100, 2
    y = torch.full((B, N), 7.0, dtype=torch.bfloat16, device=G.dev())
    z8 = torch.zeros(1, dtype=torch.uint8, device=G.dev())
    z32 = torch.zeros(1, dtype=torch.float32, device=G.dev())
    nf4.nf4_gemv_absmax32(z8, z32, N, 0, torch.zeros((B, 0), dtype=torch.bfloat16,
                                                     device=G.dev()), y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# ---------------------------------------------------------------------------
# GEMV past 2^31 weights (both formats), sampled rows
# ---------------------------------------------------------------------------

BIG_K = 4096
BIG_N = (1 << 31) // BIG_K + 64          # N * K just above 2^31
ROWS_PER_GROUP = 16384 // BIG_K          # rows that share one absmax2 group


@pytest.mark.parametrize("fmt", ["double", "absmax32"])
@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_past_2g_weights_sampled_rows(fmt, batch):
    """Random codes and scales generated on the device; the oracle checks 64
    rows taken as 16 whole absmax2 groups, so that the block and group indices
    of the extracted rows are those of the full matrix."""
    N, K = BIG_N, BIG_K
    n = N * K
    assert n >= 1 << 31
    gen = torch.Generator(device=G.dev())
    gen.manual_seed(500 + batch)
    packed = torch.randint(0, 256, (n // 2,), dtype=torch.uint8, device=G.dev(), generator=gen)
    nb = n // 64
    rng = np.random.default_rng(600 + batch)
    xbits = synth.activations(700 + batch, batch, K)
    x = G.x_to_device(xbits)
    y = torch.empty((batch, N), dtype=torch.bfloat16, device=G.dev())
    quads = np.sort(rng.choice(N // ROWS_PER_GROUP, 16, replace=False))
    rows = (quads[:, None] * ROWS_PER_GROUP + np.arange(ROWS_PER_GROUP)).reshape(-1)
    qsel = torch.from_numpy(quads).to(G.dev())
    per_g = ROWS_PER_GROUP * K
    sub_packed = packed.view(-1, per_g // 2)[qsel].cpu().numpy().reshape(-1)
    print(f"[gemv_past_2g] fmt={fmt} N={N} K={K} B={batch}", flush=True)
    if fmt == "double":
        absmax_q = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=G.dev(), generator=gen)
        a2 = (rng.standard_normal(nb // 256) * 0.05).astype(np.float16)
        code2 = oracle.code2_linear()
        nf4.nf4_gemv(packed, absmax_q, G.h16(a2.view(np.uint16)), G.h16(code2), 0.01, N, K, x,
                     64, 256, y=y)
        sub = oracle.Quantized(sub_packed, absmax_q.view(-1, per_g // 64)[qsel].cpu().numpy()
                               .reshape(-1), a2.view(np.uint16)[quads], code2,
                               float(np.float32(0.01)), rows.size * K, 64, 256)
        yr, S = oracle.gemv(sub, rows.size, K, xbits)
    else:
        absmax = torch.randn(nb, dtype=torch.float32, device=G.dev(), generator=gen) * 0.05
        nf4.nf4_gemv_absmax32(packed, absmax, N, K, x, 64, y=y)
        sub = oracle.QuantizedSL(sub_packed, absmax.view(-1, per_g // 64)[qsel].cpu().numpy()
                                 .reshape(-1), rows.size * K, 64)
        yr, S = oracle.gemv_sl(sub, rows.size, K, xbits)
    torch.cuda.synchronize()
    got = G.bf16_to_f64(G.bits16(y[:, torch.from_numpy(rows).to(G.dev())]))
    ok, worst = G.gemv_within_tolerance(got, yr, S)
    assert ok, f"worst error/bound = {worst:.3g}"
    del packed
    torch.cuda.empty_cache()
