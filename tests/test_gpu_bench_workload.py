"""GPU parity of the headline workload exactly as bench.py times it: the
32-layer 7B-shaped decode sweep (224 batch-1 GEMVs, weights drawn and encoded
on the GPU by nf4_quantize) run as one grouped launch per K with the
scheduling workspace (bench.make_step, stream schedule), plus the standalone
dequant of the 8192 x 28672 weight.  Outputs are checked against the oracle on
the device-encoded data: every GEMV (layer 0 in full, 64 random rows of each
of the others) within the rule of tests/_gpu.py, the dequant bit for bit on
sampled elements."""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def workload():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nf4.load()
    print("[bench_workload] encoding the 224 sweep matrices and the 8192x28672 weight on the GPU",
          flush=True)
    wl = bench.build_workload(G.dev())
    yield wl
    del wl
    torch.cuda.empty_cache()


def _host_q(t):
    return oracle.Quantized(t.packed.cpu().numpy(), t.absmax_q.cpu().numpy(),
                            t.absmax2.cpu().numpy().view(np.uint16),
                            t.code2.cpu().numpy().view(np.uint16), t.offset, t.n)


def test_sweep_grouped_launches_match_oracle(workload):
    """Every one of the 224 GEMVs is checked: all rows of layer 0's seven
    matrices, and 64 random rows of each matrix of the other 31 layers."""
    wl = workload
    gemvs, _, launches = bench.make_step(wl, "stream")
    assert launches == 2
    for mats in wl["layers"]:
        for (_, _, y, _) in mats:
            y.fill_(float("nan"))
    print("[bench_workload] two grouped launches (K=4096: 192 matrices, K=11008: 32)", flush=True)
    gemvs()
    torch.cuda.synchronize()
    # every output of all 224 matrices was written
    for L, mats in enumerate(wl["layers"]):
        for (g, _, y, _) in mats:
            assert bool(torch.isfinite(y).all()), f"layer {L} {g.name}: unwritten or non-finite y"
    rng = np.random.default_rng(2024)
    checked_matrices, checked_rows = 0, 0
    for L, mats in enumerate(wl["layers"]):
        for (g, t, y, x) in mats:
            rows = np.arange(g.N) if L == 0 else np.sort(rng.choice(g.N, 64, replace=False))
            xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
            yr, S = oracle.gemv(_host_q(t), g.N, g.K, xb, rows)
            got = G.bf16_to_f64(G.bits16(y)).reshape(1, g.N)[:, rows]
            ok, worst = G.gemv_within_tolerance(got, yr, S)
            assert ok, f"layer {L} {g.name}: worst error/bound = {worst:.3g}"
            checked_matrices += 1
            checked_rows += rows.size
        if L % 8 == 7:
            print(f"[bench_workload] layers 0-{L} checked", flush=True)
    assert checked_matrices == 224
    print(f"[bench_workload] {checked_matrices} GEMVs, {checked_rows} rows within tolerance",
          flush=True)


def test_big_dequant_as_benchmarked(workload):
    big, tb, out = workload["big"]
    out.fill_(float("nan"))
    tb.dequant(out=out)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(7).choice(big.n, 1 << 16, replace=False))
    idx = np.concatenate([idx, np.arange(big.n - 64, big.n)])
    got = G.bits16(out)[idx]
    ref = oracle.dequant_at(_host_q(tb), idx, oracle.BF16)
    assert np.array_equal(got, ref), f"{int(np.sum(got != ref))} of {idx.size} sampled elements differ"
