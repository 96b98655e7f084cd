"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Dequant must be bit-exact for every element, including the sign of zero.
GEMV outputs (bf16) must each be the round-to-nearest-even bf16 value of some
real within 2^-14 sum_k |w x| of the fp64 oracle result (tests/_gpu.py); this
implies |y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) 2^-14 sum_k |w x|.  Output
buffers sit between guard regions that must come back untouched.
"""
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


def run_dequant(q, out_dtype=oracle.BF16, offset_elems=0, packed_offset=0):
    d = G.fmt_to_device(q)
    if packed_offset:
        buf = torch.zeros(q.packed.size + packed_offset, dtype=torch.uint8, device=G.dev())
        buf[packed_offset:] = d["packed"]
        d["packed"] = buf[packed_offset:]
    base, out = G.guarded(q.n, DT[out_dtype], offset_elems)
    print(f"[dequant] n={q.n} bs={q.blocksize} s2={q.s2_blocksize} dtype={out_dtype} "
          f"out_off={offset_elems} packed_off={packed_offset}", flush=True)
    nf4.nf4_dequant(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, q.n,
                    q.blocksize, q.s2_blocksize, out=out)
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

def test_dequant_1024x1024_bf16():
    cfg = synth.DEQUANT_1K
    q = oracle.quantize(synth.weights(cfg.seed, cfg.n))
    assert_bits_equal(run_dequant(q, oracle.BF16), oracle.dequant(q, oracle.BF16))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_dequant_4096x4096_outliers(dtype):
    cfg = synth.DEQUANT_4K
    q = oracle.quantize(synth.weights(cfg.seed, cfg.n, outliers=True))
    assert_bits_equal(run_dequant(q, dtype), oracle.dequant(q, dtype))


EDGE = [
    (1, 64, 256), (2, 64, 256), (7, 64, 256), (8, 64, 256), (9, 64, 256), (63, 64, 256),
    (65, 64, 256), (12345, 64, 256), (2047 * 4096, 64, 256), (64 * 256 * 3 + 64, 64, 256),
    (100_003, 64, 256), (2048 * 8 * 3 + 5, 64, 256), (4096, 8, 2), (4099, 16, 1),
    (5000, 32, 4), (5000, 128, 256), (3001, 4, 8), (3001, 2, 1), (777, 1, 4),
    (70_000, 1 << 14, 1), (1 << 16, 64, 1 << 12),
    # tile-size boundaries of the vector path on 256 CUs: 1, 2 and 4 steps
    # per lane, each with a ragged tail; blocksize 8 fills the scale table
    (1_048_575, 64, 256), (1_500_001, 64, 256), (2_097_147, 64, 256), (2_100_003, 8, 2),
]


@pytest.mark.parametrize("n,bs,s2", EDGE)
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_dequant_edge_shapes(n, bs, s2, dtype):
    q = oracle.quantize(synth.weights(n + bs + s2, n, outliers=True), bs, s2)
    assert_bits_equal(run_dequant(q, dtype), oracle.dequant(q, dtype))


@pytest.mark.parametrize("offset_elems,packed_offset", [(1, 0), (0, 1), (3, 2), (4, 0)])
def test_dequant_unaligned_buffers(offset_elems, packed_offset):
    q = oracle.quantize(synth.weights(31, 50_001))
    for dtype in (oracle.BF16, oracle.FP16):
        assert_bits_equal(run_dequant(q, dtype, offset_elems, packed_offset),
                          oracle.dequant(q, dtype))


def _hand_format(n, bs, s2, code2_vals, absmax2_vals, absmax_q, packed, offset):
    return oracle.Quantized(np.ascontiguousarray(packed, np.uint8),
                            np.ascontiguousarray(absmax_q, np.uint8),
                            np.asarray(absmax2_vals, np.float16).view(np.uint16),
                            np.asarray(code2_vals, np.float16).view(np.uint16),
                            float(np.float32(offset)), n, bs, s2)


@pytest.mark.parametrize("case", ["neg_zero", "subnormal", "huge", "random_scales"])
def test_dequant_special_values(case):
    """Negative absmax_real (zero code -> -0), results in the subnormal range
    of bf16/fp16, fp16 overflow, and random fp16 scales over many binades:
    rounding on the GPU must match the oracle's round-to-nearest-even."""
    rng = np.random.default_rng({"neg_zero": 1, "subnormal": 2, "huge": 3, "random_scales": 4}[case])
    n, bs, s2 = 64 * 1024, 64, 4
    nb, ng = n // bs, n // bs // s2
    packed = rng.integers(0, 256, n // 2).astype(np.uint8)
    absmax_q = rng.integers(0, 256, nb).astype(np.uint8)
    if case == "neg_zero":
        q = _hand_format(n, bs, s2, np.full(256, -1.0), np.ones(ng), absmax_q,
                         np.full(n // 2, 0x77, np.uint8), 0.25)
    elif case == "subnormal":
        code2 = rng.standard_normal(256) * 2.0 ** -14
        code2[:16] = 0.0          # absmax_real = offset: bf16 subnormal outputs
        q = _hand_format(n, bs, s2, code2, 2.0 ** -rng.integers(5, 14, ng), absmax_q, packed,
                         -1e-39)
    elif case == "huge":
        q = _hand_format(n, bs, s2, rng.uniform(-1, 1, 256) * 60000, rng.uniform(0.5, 2.0, ng),
                         absmax_q, packed, 3e4)
    else:
        code2 = rng.standard_normal(256) * 2.0 ** rng.integers(-12, 4, 256)
        a2 = rng.standard_normal(ng) * 2.0 ** rng.integers(-12, 8, ng)
        q = _hand_format(n, bs, s2, code2, a2, absmax_q, packed, rng.standard_normal() * 1e-3)
    for dtype in (oracle.BF16, oracle.FP16):
        with np.errstate(over="ignore"):
            assert_bits_equal(run_dequant(q, dtype), oracle.dequant(q, dtype))


def test_dequant_8192x28672():
    cfg = synth.DEQUANT_BIG
    q = oracle.quantize(synth.weights(cfg.seed, cfg.n))
    assert_bits_equal(run_dequant(q, oracle.BF16), oracle.dequant(q, oracle.BF16))


def test_dequant_is_deterministic():
    q = oracle.quantize(synth.weights(77, 1 << 20))
    a = run_dequant(q)
    b = run_dequant(q)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def run_gemv(q, N, K, xbits, x_offset=0):
    d = G.fmt_to_device(q)
    B = xbits.shape[0]
    x = G.x_to_device(xbits)
    if x_offset:
        buf = torch.zeros(B * K + x_offset, dtype=torch.bfloat16, device=G.dev())
        buf[x_offset:] = x.reshape(-1)
        x = buf[x_offset:].view(B, K)
    base, yv = G.guarded(B * N, torch.bfloat16)
    print(f"[gemv] N={N} K={K} B={B} bs={q.blocksize} s2={q.s2_blocksize} x_off={x_offset}",
          flush=True)
    nf4.nf4_gemv(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, N, K, x,
                 q.blocksize, q.s2_blocksize, y=yv.view(B, N))
    torch.cuda.synchronize()
    assert G.guards_intact(base, B * N), "write outside y"
    return G.bf16_to_f64(G.bits16(yv)).reshape(B, N)


def check_gemv(q, N, K, xbits, rows=None, x_offset=0):
    y = run_gemv(q, N, K, xbits, x_offset)
    yr, S = oracle.gemv(q, N, K, xbits, rows)
    if rows is not None:
        y = y[:, rows]
    ok, worst = G.gemv_within_tolerance(y, yr, S)
    assert ok, f"GEMV N={N} K={K} B={xbits.shape[0]}: worst error/bound = {worst:.3g}"
    return worst


@pytest.mark.parametrize("g", synth.QWEN_GEMVS, ids=lambda g: g.name)
def test_gemv_qwen_batch1(g):
    q = oracle.quantize(synth.weights(g.seed, g.N * g.K))
    check_gemv(q, g.N, g.K, synth.activations(synth.QWEN_X_SEED, 1, g.K))


@pytest.mark.parametrize("batch", synth.LLAMA_BATCHES)
@pytest.mark.parametrize("g", synth.LLAMA_GEMVS, ids=lambda g: g.name)
def test_gemv_llama(g, batch):
    q = oracle.quantize(synth.weights(g.seed, g.N * g.K))
    check_gemv(q, g.N, g.K, synth.activations(synth.llama_x_seed(batch), batch, g.K))


@pytest.mark.parametrize("g", synth.sweep_layer(0), ids=lambda g: g.name)
def test_gemv_decode_sweep_layer0(g):
    q = oracle.quantize(synth.weights(g.seed, g.N * g.K))
    rows = np.random.default_rng(g.seed).choice(g.N, 512, replace=False)
    check_gemv(q, g.N, g.K, synth.activations(synth.SWEEP_X_SEED, 1, g.K), rows=np.sort(rows))


GEMV_EDGE = [
    # N, K, bs, s2
    (1, 64, 64, 256), (3, 64, 64, 256), (5, 2048, 64, 256), (7, 2080, 64, 256),
    (33, 32, 32, 1), (17, 96, 32, 4), (9, 16384, 64, 256), (3, 16416, 64, 256),
    (11, 1000, 64, 256), (13, 2, 64, 256), (6, 130, 2, 8), (300, 1536, 128, 2),
    (257, 1536, 16, 256), (64, 4096, 1 << 12, 1), (2, 40000, 64, 256),
    # an 8-way shard of a 4096 -> 11008 projection (rows) and of 11008 -> 4096 (columns)
    (1376, 4096, 64, 256), (4096, 1376, 64, 256),
    # two and three 4096-column passes per wave, at their upper ends
    (100, 8192, 64, 256), (50, 12288, 64, 256), (40, 12352, 64, 256),
    # one 64-column block past a wave load's start: only lanes 0 and 1 of the
    # second load (2112) or of the second pass's first load (4160) hold columns
    (21, 2112, 64, 256), (19, 4160, 128, 2),
]


@pytest.mark.parametrize("N,K,bs,s2", GEMV_EDGE)
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
def test_gemv_edge_shapes(N, K, bs, s2, batch):
    q = oracle.quantize(synth.weights(N * 7 + K, N * K, outliers=True), bs, s2)
    check_gemv(q, N, K, synth.activations(N + K + batch, batch, K))


# One matrix at batch 3-8 with K <= 4096 takes the fp32-product team kernel
# (16 columns per lane, one row per group at batch 3-4, two at 5-8): slabs cut
# short by K, row counts that leave a group half empty, and small blocks.
GEMV_FP32_PRODUCTS = [
    # N, K, bs, s2
    (37, 4096, 64, 256), (130, 1056, 32, 4), (9, 64, 64, 256), (515, 3072, 128, 2),
    (2, 2048, 64, 1), (1, 4096, 4096, 1),
]


@pytest.mark.parametrize("N,K,bs,s2", GEMV_FP32_PRODUCTS)
@pytest.mark.parametrize("batch", [3, 4, 5, 6, 7, 8])
def test_gemv_fp32_products_batch3_to_8(N, K, bs, s2, batch):
    q = oracle.quantize(synth.weights(N * 11 + K + 3, N * K, outliers=True), bs, s2)
    check_gemv(q, N, K, synth.activations(N + 3 * K + batch, batch, K))


@pytest.mark.parametrize("scale", [1e-36, 1e-39])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv_tiny_activations(scale, batch):
    """Activations near and below the smallest normal bf16 (1e-39: most are
    bf16 subnormals, and so are the outputs): the dot2 decode (batch 1-2) and
    the fp32-product decode (batch 4, 8) both stay within the bf16 rounding
    of the tolerance band (on the subnormal grid that band is wide in
    relative terms)."""
    N, K = 64, 4096
    q = oracle.quantize(synth.weights(5, N * K))
    xf = (np.random.default_rng(batch).standard_normal((batch, K)) * scale).astype(np.float32)
    xb = oracle.bf16_from_f32(xf).reshape(batch, K)
    y = run_gemv(q, N, K, xb)
    yr, S = oracle.gemv(q, N, K, xb, None)
    ok, _ = G.gemv_within_tolerance(y, yr, S)
    assert ok, f"scale {scale} batch {batch}"
    assert np.count_nonzero(yr) > 0


@pytest.mark.parametrize("batch", [1, 4, 6, 7, 8])
def test_gemv_unaligned_x(batch):
    N, K = 40, 4096
    q = oracle.quantize(synth.weights(5, N * K))
    check_gemv(q, N, K, synth.activations(6, batch, K), x_offset=1)


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv_one_hot_picks_the_column(batch):
    """x = e_k in every batch row: y[r] is a single product, the fp32 dequant
    value W[r][k] up to the decode table's 2^-16 (G.one_hot_ok) -- no
    accumulation error, and every row, column and batch index checked."""
    N, K = 256, 4096
    q = oracle.quantize(synth.weights(8, N * K))
    W = oracle.dequant_f32(q).reshape(N, K)
    ks = [0, 31, 32, 2047, 2048, 4095][:batch] + [1000] * max(0, batch - 6)
    x = np.zeros((batch, K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    y = run_gemv(q, N, K, synth.to_bf16_bits(x))
    for b, k in enumerate(ks):
        assert G.one_hot_ok(y[b], W[:, k]), f"batch row {b}, k={k}"


def test_gemv_empty_k_gives_zeros():
    N, B = 100, 3
    y = torch.full((B, N), 7.0, dtype=torch.bfloat16, device=G.dev())
    z8 = torch.zeros(1, dtype=torch.uint8, device=G.dev())
    z16 = torch.zeros(256, dtype=torch.int16, device=G.dev())
    x = torch.zeros((B, 0), dtype=torch.bfloat16, device=G.dev())
    nf4.nf4_gemv(z8, z8, z16, z16, 0.0, N, 0, x, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_gemv_is_deterministic():
    N, K, B = 4096, 4096, 4
    q = oracle.quantize(synth.weights(9, N * K))
    xb = synth.activations(10, B, K)
    a = run_gemv(q, N, K, xb)
    b = run_gemv(q, N, K, xb)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# grouped GEMV (one launch over several matrices)
# ---------------------------------------------------------------------------

def _group_case(shapes_seeds, K, batch, x_seed):
    qs, items, ys = [], [], []
    for N, seed in shapes_seeds:
        q = oracle.quantize(synth.weights(seed, N * K))
        d = G.fmt_to_device(q)
        w = nf4.NF4Tensor(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, q.n)
        xb = synth.activations(x_seed + seed, batch, K)
        base, yv = G.guarded(batch * N, torch.bfloat16)
        items.append((w, N, G.x_to_device(xb), yv.view(batch, N)))
        qs.append((q, N, xb, base))
    return qs, items


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("K,shapes", [
    (4096, [(4096, 600), (4096, 601), (11008, 602), (256, 603), (1, 604), (37, 605)]),
    (1536, [(1536, 610), (256, 611), (256, 612), (8960, 613)]),
    (11008, [(4096, 620), (3, 621)]),
    # two 4096-column passes per wave; three at their upper end; one column
    # block past it (no wave configuration: the team kernel)
    (8192, [(300, 640), (7, 641)]),
    (12288, [(40, 650), (9, 651)]),
    (12352, [(33, 655), (2, 656)]),
    (96, [(5, 630), (3, 631)]),
])
def test_gemv_grouped_matches_oracle(K, shapes, batch):
    qs, items = _group_case(shapes, K, batch, 700)
    grp = nf4.GemvGroup(items, K)
    print(f"[gemv_grouped] K={K} B={batch} N={[n for n, _ in shapes]}", flush=True)
    grp.launch()
    torch.cuda.synchronize()
    for (q, N, xb, base), (_, _, _, yv) in zip(qs, items):
        assert G.guards_intact(base, batch * N), "write outside y"
        y = G.bf16_to_f64(G.bits16(yv)).reshape(batch, N)
        yr, S = oracle.gemv(q, N, K, xb)
        ok, worst = G.gemv_within_tolerance(y, yr, S)
        assert ok, f"grouped N={N} K={K}: worst {worst:.3g}"


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 11008), (11008, 4096), (1536, 256)])
def test_gemv_group_of_one_matrix(K, N, batch):
    """A group of one matrix launches through nf4_gemv (its descriptor in the
    kernel arguments): the same bits as nf4_gemv called directly, within
    tolerance of the oracle; nf4_gemv_grouped on the group's uploaded table
    (the grouped kernels) meets the oracle too."""
    qs, items = _group_case([(N, 690)], K, batch, 795)
    grp = nf4.GemvGroup(items, K)
    assert grp.single is not None and grp.sched is None
    (q, _, xb, base), (w, _, x, yv) = qs[0], items[0]
    print(f"[gemv_group_of_one] K={K} N={N} B={batch}", flush=True)
    yv.fill_(float("nan"))
    grp.launch()
    torch.cuda.synchronize()
    y_group = G.bits16(yv).copy()
    yv.fill_(float("nan"))
    w.gemv(N, K, x, yv)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits16(yv), y_group), "group of one differs from nf4_gemv"
    yv.fill_(float("nan"))
    st = nf4.load().nf4_gemv_grouped(grp.table.data_ptr(), 1, N, K, 64, 256,
                                     w.code2.data_ptr(), batch, None, 0,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    y_grouped = G.bits16(yv).copy()
    assert G.guards_intact(base, batch * N), "write outside y"
    yr, S = oracle.gemv(q, N, K, xb)
    for name, bits in (("group of one", y_group), ("grouped kernels", y_grouped)):
        y = G.bf16_to_f64(bits).reshape(batch, N)
        ok, worst = G.gemv_within_tolerance(y, yr, S)
        assert ok, f"{name} N={N} K={K} B={batch}: worst {worst:.3g}"


def test_gemv_grouped_dynamic_schedule():
    """Enough rows (>= 64 per wave) for chunked row distribution: the
    results match the oracle, are bit-identical to the fixed split, stay the
    same over repeated launches, and every launch leaves the workspace at
    zero."""
    K = 128
    shapes = [(100003, 680), (150001, 681), (50000, 682)]
    qs, items = _group_case(shapes, K, 1, 790)
    ys_static = [torch.empty_like(it[3]) for it in items]
    grp = nf4.GemvGroup(items, K, dynamic=True)
    ref = nf4.GemvGroup([(w, N, x, ys) for (w, N, x, _), ys in zip(items, ys_static)], K,
                        dynamic=False)
    assert grp.sched is not None and ref.sched is None
    print(f"[gemv_grouped_dynamic] K={K} rows={sum(n for n, _ in shapes)}", flush=True)
    ref.launch()
    first = None
    for rep in range(3):
        for it in items:
            it[3].fill_(float("nan"))
        grp.launch()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(grp.sched)) == 0, f"workspace not reset after launch {rep}"
        ys = [it[3].view(torch.int16).clone() for it in items]
        if first is None:
            first = ys
        for a, b in zip(ys, first):
            assert torch.equal(a, b), f"launch {rep} differs from launch 0"
    for a, b in zip(first, ys_static):
        assert torch.equal(a, b.view(torch.int16)), "dynamic and fixed split differ"
    for (q, N, xb, base), (_, _, _, yv) in zip(qs, items):
        assert G.guards_intact(base, N), "write outside y"
        y = G.bf16_to_f64(G.bits16(yv)).reshape(1, N)
        yr, S = oracle.gemv(q, N, K, xb)
        ok, worst = G.gemv_within_tolerance(y, yr, S)
        assert ok, f"dynamic N={N}: worst {worst:.3g}"


def test_gemv_grouped_skips_bad_descriptors():
    """A descriptor whose N disagrees with the row offsets is skipped: its y
    keeps its old contents; the others are still computed."""
    import numpy as np
    K = 512
    qs, items = _group_case([(64, 640), (32, 641)], K, 1, 750)
    grp = nf4.GemvGroup(items, K)
    tab = grp.table.cpu().numpy().copy().view(np.int64).reshape(len(items), 8)
    tab[1, 5] = 31                                    # N of item 1 no longer matches
    grp.table.copy_(torch.from_numpy(tab.view(np.uint8).reshape(-1)))
    items[1][3].fill_(3.0)
    grp.launch()
    torch.cuda.synchronize()
    assert torch.all(items[1][3] == 3.0)
    q, N, xb, base = qs[0]
    y = G.bf16_to_f64(G.bits16(items[0][3])).reshape(1, N)
    yr, S = oracle.gemv(q, N, K, xb)
    assert G.gemv_within_tolerance(y, yr, S)[0]


@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("K", [8192, 11008, 16384])
def test_gemv_grouped_many_small_matrices(K, batch):
    """More than one pass, many matrices of 1-9 rows with their own
    activations, and every tenth of 700-900 rows so that the launch has rows
    enough for the shared-activation kernel: a workgroup's row range crosses
    many matrices, so the activations are staged again for each one; a matrix
    with a bad N in the middle is skipped (its y keeps its contents) and the
    others are computed."""
    import numpy as np
    rng = np.random.default_rng(K + batch)
    sizes = rng.integers(1, 10, size=120)
    sizes[::10] = rng.integers(700, 900, size=12)
    shapes = [(int(n), 900 + i) for i, n in enumerate(sizes)]
    shapes[41] = (5, 940)
    qs, items = [], []
    for N, seed in shapes:
        q = oracle.quantize(synth.weights(seed, N * K))
        d = G.fmt_to_device(q)
        w = nf4.NF4Tensor(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, q.n)
        xb = synth.activations(seed + 7, batch, K)
        base, yv = G.guarded(batch * N, torch.bfloat16)
        items.append((w, N, G.x_to_device(xb), yv.view(batch, N)))
        qs.append((q, N, xb, base))
    grp = nf4.GemvGroup(items, K)
    tab = grp.table.cpu().numpy().copy().view(np.int64).reshape(len(items), 8)
    tab[41, 5] = 4                                    # N of item 41 no longer matches
    grp.table.copy_(torch.from_numpy(tab.view(np.uint8).reshape(-1)))
    items[41][3].fill_(3.0)
    print(f"[gemv_grouped_many] K={K} B={batch} matrices={len(shapes)} rows={grp.total_rows}",
          flush=True)
    grp.launch()
    torch.cuda.synchronize()
    assert grp.total_rows >= 2 * 16 * 256, "too few rows for the shared-activation kernel"
    assert torch.all(items[41][3] == 3.0), "the bad matrix was written"
    for i, ((q, N, xb, base), (_, _, _, yv)) in enumerate(zip(qs, items)):
        assert G.guards_intact(base, batch * N), f"write outside y of item {i}"
        if i == 41:
            continue
        y = G.bf16_to_f64(G.bits16(yv)).reshape(batch, N)
        yr, S = oracle.gemv(q, N, K, xb)
        ok, worst = G.gemv_within_tolerance(y, yr, S)
        assert ok, f"item {i} N={N}: worst {worst:.3g}"


def test_graph_replay_matches_eager():
    """A HIP graph holding a grouped GEMV and a dequant, replayed several
    times with eager work and synchronizations in between, reproduces the
    eager results bit for bit on every replay."""
    K = 1024
    qs, items = _group_case([(512, 660), (96, 661)], K, 1, 770)
    grp = nf4.GemvGroup(items, K)
    q = oracle.quantize(synth.weights(662, 1 << 18))
    d = G.fmt_to_device(q)
    out = torch.empty(q.n, dtype=torch.bfloat16, device=G.dev())

    def step():
        grp.launch()
        nf4.nf4_dequant(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, q.n, out=out)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref_y = [it[3].clone() for it in items]
    ref_out = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for it in items:
            it[3].fill_(-1.0)
        out.fill_(-2.0)
        junk = torch.randn(1 << 20, device=G.dev()).sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for it, r in zip(items, ref_y):
            assert torch.equal(it[3].view(torch.int16), r.view(torch.int16)), f"replay {rep}"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}"
