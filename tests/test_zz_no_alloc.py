"""GPU test of nf4_gemv_grouped_noalloc, the grouped GEMV that allocates
nothing (its scheduling counters live in the library's per-GPU scratch).

Through the C ABI, two no-allocation launches in a row -- the second over a
smaller input, so it runs on the scratch the first one left behind -- must give
bit for bit the outputs of nf4_gemv_grouped with a caller-provided scheduling
workspace and with the fixed split.  Both inputs are large enough that the
launch hands out rows in chunks (>= 64 rows per wave of the largest grid), so
the scratch is really used; 64 sampled rows of one matrix per launch are also
checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu

K = 4096
ROWS = 4096            # rows per matrix
OFFSET = 0.0371


def _random_group(n_mats, seed):
    """n_mats random NF4 matrices [ROWS][K] (random codes and scales drawn on the
    GPU) sharing one x, with a y each."""
    dev = G.dev()
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    n = ROWS * K
    nb, ng = n // 64, n // (64 * 256)
    packed = torch.randint(0, 256, (n_mats, n // 2), generator=g, device=dev, dtype=torch.uint8)
    absmax_q = torch.randint(0, 256, (n_mats, nb), generator=g, device=dev, dtype=torch.uint8)
    absmax2 = (torch.rand(n_mats, ng, generator=g, device=dev) * 0.05 + 1e-3).half() \
        .view(torch.int16)
    x = torch.randn(1, K, generator=g, device=dev).to(torch.bfloat16)
    code2 = nf4.nf4_code2_linear().to(dev)
    mats = [nf4.NF4Tensor(packed[i], absmax_q[i], absmax2[i], code2, OFFSET, n)
            for i in range(n_mats)]
    ys = [torch.empty(1, ROWS, dtype=torch.bfloat16, device=dev) for _ in range(n_mats)]
    return mats, x, ys


def _run(mats, x, ys, **kw):
    for y in ys:
        y.fill_(float("nan"))
    grp = nf4.GemvGroup([(t, ROWS, x, y) for t, y in zip(mats, ys)], K, **kw)
    grp.launch()
    return grp


def _oracle_rows(t, x, y, seed):
    rows = np.sort(np.random.default_rng(seed).choice(ROWS, 64, replace=False))
    q = oracle.Quantized(t.packed.cpu().numpy(), t.absmax_q.cpu().numpy(),
                         t.absmax2.cpu().numpy().view(np.uint16),
                         t.code2.cpu().numpy().view(np.uint16), t.offset, t.n)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    yr, S = oracle.gemv(q, ROWS, K, xb, rows)
    got = G.bf16_to_f64(G.bits16(y)).reshape(1, ROWS)[:, rows]
    return G.gemv_within_tolerance(got, yr, S)


def test_noalloc_grouped_matches_the_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nf4.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # chunked scheduling needs >= 64 rows per wave of the 2-per-CU grid
    need = 64 * 8 * 2 * cus
    sizes = (need // ROWS + 6, need // ROWS + 2)          # the second launch is smaller
    assert sizes[1] * ROWS >= need and sizes[1] < sizes[0]
    cases = []
    for i, n_mats in enumerate(sizes):
        print(f"[no_alloc] building {n_mats} matrices of {ROWS}x{K}", flush=True)
        mats, x, ys = _random_group(n_mats, 77 + i)
        keep = []
        refs = {}
        for name, kw in (("workspace", dict(dynamic=True)), ("fixed", dict(dynamic=False))):
            keep.append(_run(mats, x, ys, **kw))
            torch.cuda.synchronize()
            refs[name] = [G.bits16(y).copy() for y in ys]
        cases.append((mats, x, ys, refs, keep))
    # the two no-allocation launches, back to back on one stream
    groups = []
    for i, (mats, x, ys, _, _) in enumerate(cases):
        print(f"[no_alloc] launch {i}: {len(mats)} matrices", flush=True)
        for y in ys:
            y.fill_(float("nan"))
        groups.append(nf4.GemvGroup([(t, ROWS, x, y) for t, y in zip(mats, ys)], K,
                                    noalloc=True))
    outs = []
    for i, (grp, (mats, x, ys, _, _)) in enumerate(zip(groups, cases)):
        grp.launch()
        torch.cuda.synchronize()
        outs.append([G.bits16(y).copy() for y in ys])
    for i, ((mats, x, ys, refs, _), out) in enumerate(zip(cases, outs)):
        for name, ref in refs.items():
            for j, (a, b) in enumerate(zip(out, ref)):
                assert np.array_equal(a, b), f"launch {i}, matrix {j}: differs from the {name} run"
        ok, worst = _oracle_rows(mats[-1], x, ys[-1], 500 + i)
        assert ok, f"launch {i}: worst error/bound = {worst:.3g}"
    print(f"[no_alloc] {sizes[0]} and {sizes[1]} matrices bit-identical to nf4_gemv_grouped",
          flush=True)
