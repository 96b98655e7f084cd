"""GPU parity for nf4_gemm, the batched product on the matrix cores (batch
rows past 8, prefill), through the C ABI against the oracle's fp64 GEMV on
the same seeded inputs.  Outputs must meet the GEMV rule of tests/_gpu.py
(bf16 rounding of a value within 2^-14 sum |w x| of the fp64 result); the
output buffer sits between guard regions."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nf4.load()


def run_gemm(q, N, K, xbits, x_offset=0, workspace="auto"):
    """workspace: "auto" (a fresh zeroed one of nf4_gemm_workspace_size bytes),
    None, or a tensor to reuse."""
    M = xbits.shape[0]
    d = G.fmt_to_device(q)
    x = G.x_to_device(xbits)
    if x_offset:
        buf = torch.zeros(M * K + x_offset, dtype=torch.bfloat16, device=G.dev())
        buf[x_offset:] = x.reshape(-1)
        x = buf[x_offset:].view(M, K)
    base, yv = G.guarded(M * N, torch.bfloat16)
    if isinstance(workspace, str):
        workspace = nf4.nf4_gemm_workspace(M, N, K)
    wsb = 0 if workspace is None else workspace.numel()
    print(f"[gemm] M={M} N={N} K={K} bs={q.blocksize} s2={q.s2_blocksize} x_off={x_offset} "
          f"workspace={wsb}", flush=True)
    nf4.nf4_gemm(d["packed"], d["absmax_q"], d["absmax2"], d["code2"], q.offset, N, K, x,
                 q.blocksize, q.s2_blocksize, y=yv.view(M, N), workspace=workspace)
    torch.cuda.synchronize()
    assert G.guards_intact(base, M * N), "write outside y"
    return G.bf16_to_f64(G.bits16(yv)).reshape(M, N)


def check_gemm(q, N, K, xbits, rows=None, x_offset=0, workspace="auto"):
    y = run_gemm(q, N, K, xbits, x_offset, workspace)
    yr, S = oracle.gemv(q, N, K, xbits, rows)
    if rows is not None:
        y = y[:, rows]
    ok, worst = G.gemv_within_tolerance(y, yr, S)
    assert ok, f"GEMM M={xbits.shape[0]} N={N} K={K}: worst error/bound = {worst:.3g}"


@pytest.mark.parametrize("M", [16, 64, 128])
@pytest.mark.parametrize("g", synth.LLAMA_GEMVS, ids=lambda g: g.name)
def test_gemm_llama(g, M):
    q = oracle.quantize(synth.weights(g.seed, g.N * g.K))
    rows = np.sort(np.random.default_rng(g.seed + M).choice(g.N, 256, replace=False))
    check_gemm(q, g.N, g.K, synth.activations(600 + M, M, g.K), rows=rows)


GEMM_EDGE = [
    # M, N, K, bs, s2
    (1, 64, 4096, 64, 256), (9, 100, 4096, 64, 256), (17, 17, 1536, 64, 256),
    (33, 257, 1536, 128, 2), (50, 16, 64, 64, 1), (65, 1, 128, 64, 256), (130, 33, 192, 64, 4),
    (16, 1376, 4096, 64, 256), (24, 4096, 1376 * 2, 256, 256), (40, 300, 8192, 64, 256),
    # fallbacks: K % 64 != 0, blocksize 32, tiny K
    (20, 50, 96, 32, 4), (12, 40, 1000, 8, 256), (10, 7, 2, 64, 256),
]


@pytest.mark.parametrize("M,N,K,bs,s2", GEMM_EDGE)
def test_gemm_edge_shapes(M, N, K, bs, s2):
    q = oracle.quantize(synth.weights(M + N + K, N * K, outliers=True), bs, s2)
    check_gemm(q, N, K, synth.activations(M * 3 + K, M, K))


def test_gemm_unaligned_x_falls_back():
    M, N, K = 20, 64, 4096
    q = oracle.quantize(synth.weights(61, N * K))
    check_gemm(q, N, K, synth.activations(62, M, K), x_offset=1)


def test_gemm_one_hot_picks_the_column():
    """x[m] = e_{k_m}: y[m][n] is the single product W[n][k_m] up to the
    decode table's 2^-16 (G.one_hot_ok)."""
    M, N, K = 48, 96, 4096
    q = oracle.quantize(synth.weights(63, N * K))
    W = oracle.dequant_f32(q).reshape(N, K)
    ks = (np.arange(M) * 97) % K
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), ks] = 1.0
    y = run_gemm(q, N, K, synth.to_bf16_bits(x))
    for m, k in enumerate(ks):
        assert G.one_hot_ok(y[m], W[:, k]), (m, k)


def test_gemm_is_deterministic_and_matches_gemv_shape():
    M, N, K = 72, 512, 4096
    q = oracle.quantize(synth.weights(64, N * K))
    xb = synth.activations(65, M, K)
    a = run_gemm(q, N, K, xb)
    b = run_gemm(q, N, K, xb)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M,N,K", [(128, 4096, 4096), (16, 4096, 11008), (40, 1376, 4096)])
def test_gemm_split_k(M, N, K):
    """With a workspace the product splits K over workgroups and sums the fp32
    partials in a fixed order: the same bits twice in a row on the same
    workspace (the second time over the first call's partials), and both the split and
    the unsplit product within the GEMV tolerance of the oracle on sampled
    columns (the split changes the fp32 summation order, so the two may differ
    in the last bits)."""
    nbytes = nf4.load().nf4_gemm_workspace_size(M, N, K)
    assert nbytes > 0, "these shapes leave compute units idle without a split"
    q = oracle.quantize(synth.weights(70 + M, N * K))
    xb = synth.activations(71 + M, M, K)
    ws = nf4.nf4_gemm_workspace(M, N, K)
    a = run_gemm(q, N, K, xb, workspace=ws)
    b = run_gemm(q, N, K, xb, workspace=ws)
    c = run_gemm(q, N, K, xb, workspace=None)
    assert np.array_equal(a, b)
    cols = np.sort(np.random.default_rng(M + N).choice(N, 96, replace=False))
    yr, S = oracle.gemv(q, N, K, xb, cols)
    for name, y in (("split", a), ("unsplit", c)):
        ok, worst = G.gemv_within_tolerance(y[:, cols], yr, S)
        assert ok, f"{name} GEMM: worst error/bound = {worst:.3g}"


@pytest.mark.parametrize("M,N,K", [
    (130, 1000, 4096),   # ragged rows (two row groups) and columns, split K
    (17, 100, 8192),     # four-block groups, ragged, split over 2^7 blocks
    (9, 4096, 11008),    # 172 blocks: splits of 43, the last group half dead
    (33, 64, 1984),      # 31 blocks: an odd count, the last pair half dead
])
def test_gemm_split_and_ragged_shapes(M, N, K):
    q = oracle.quantize(synth.weights(M + 7 * N + K, N * K, outliers=True))
    xb = synth.activations(M + K, M, K)
    cols = np.sort(np.random.default_rng(N).choice(N, min(N, 80), replace=False))
    for ws in ("auto", None):
        y = run_gemm(q, N, K, xb, workspace=ws)
        yr, S = oracle.gemv(q, N, K, xb, cols)
        ok, worst = G.gemv_within_tolerance(y[:, cols], yr, S)
        assert ok, f"M={M} N={N} K={K} ws={ws}: worst error/bound = {worst:.3g}"


def test_gemm_workspace_reused_for_a_smaller_shape():
    """A workspace sized for a larger product serves a smaller one next."""
    ws = nf4.nf4_gemm_workspace(128, 4096, 4096)
    for (M, N, K) in [(128, 4096, 4096), (24, 1024, 2048)]:
        q = oracle.quantize(synth.weights(80 + M, N * K))
        xb = synth.activations(81 + M, M, K)
        cols = np.sort(np.random.default_rng(M).choice(N, 64, replace=False))
        y = run_gemm(q, N, K, xb, workspace=ws)
        yr, S = oracle.gemv(q, N, K, xb, cols)
        ok, worst = G.gemv_within_tolerance(y[:, cols], yr, S)
        assert ok, f"M={M} N={N} K={K}: worst error/bound = {worst:.3g}"


def test_gemm_workspace_contents_do_not_matter():
    """The workspace is scratch: garbage in it changes nothing."""
    M, N, K = 128, 4096, 4096
    q = oracle.quantize(synth.weights(90, N * K))
    xb = synth.activations(91, M, K)
    ws = nf4.nf4_gemm_workspace(M, N, K)
    a = run_gemm(q, N, K, xb, workspace=ws)
    ws.fill_(0xA5)
    b = run_gemm(q, N, K, xb, workspace=ws)
    assert np.array_equal(a, b)


def test_gemm_empty_k_gives_zeros():
    M, N = 20, 30
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=G.dev())
    z8 = torch.zeros(1, dtype=torch.uint8, device=G.dev())
    z16 = torch.zeros(256, dtype=torch.int16, device=G.dev())
    nf4.nf4_gemm(z8, z8, z16, z16, 0.0, N, 0, torch.zeros((M, 0), dtype=torch.bfloat16,
                                                          device=G.dev()), y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
