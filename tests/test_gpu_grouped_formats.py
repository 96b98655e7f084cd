"""GPU parity of the grouped GEMV in the single-level format
(nf4_gemv_grouped_absmax32) and the INT4 asymmetric group format
(int4_gemv_grouped): one launch over several matrices sharing K, the block
size and the batch, through the C ABI, against the oracle's fp64 GEMV of each
matrix.  Outputs meet the rule of tests/_gpu.py (bound 2^-14 S for the
single-level format, 2^-14 M for INT4); output buffers sit between guard
regions; with and without the scheduling workspace the bits are the same."""
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


def _encode(fmt, seed, N, K, bs):
    w = synth.weights(seed, N * K, outliers=True)
    if fmt == "absmax32":
        q = oracle.quantize_sl(w, bs)
        t = nf4.NF4Absmax32Tensor(G.u8(q.packed),
                                  torch.from_numpy(q.absmax.astype(np.float32)).to(G.dev()),
                                  q.n, bs)
    else:
        q = oracle.int4_quantize(w, bs)
        t = nf4.Int4Tensor(G.u8(q.packed), G.h16(q.scales), G.h16(q.zeros), q.n, bs)
    return q, t


def _reference(fmt, q, N, K, xb):
    if fmt == "absmax32":
        yr, S = oracle.gemv_sl(q, N, K, xb)
        return yr, S
    yr, _, M = oracle.int4_gemv(q, N, K, xb)
    return yr, M


CASES = [
    # K, [(N, seed)], block (group) size
    (4096, [(4096, 900), (256, 901), (1000, 902), (1, 903)], 64),
    (4096, [(512, 904), (77, 905)], 128),
    (4096, [(8192, 906), (256, 907)], 64),         # rows enough for the shared-activation kernel
    (1536, [(1536, 910), (256, 911), (8960, 912)], 64),
    (11008, [(300, 920), (5, 921)], 64),          # three 4096-column passes
    (8192, [(200, 930), (7, 931)], 256),           # two passes
    (4160, [(64, 935), (3, 936)], 64),             # second pass: one 64-column block
    (12352, [(40, 950), (3, 951)], 64),            # four passes: the team kernel
    (96, [(33, 940), (7, 941)], 32),               # the team kernel only
]


# Several 4096-column passes with rows enough (>= 8192) for the
# shared-activation kernel, which serves these launches at batch 1-2.
XLDS_CASES = [
    (11008, [(8192, 970), (300, 971)], 64),
    (11008, [(8192, 972), (3, 973)], 128),
    (8192, [(8192, 975), (40, 976)], 64),
    (8192, [(8200, 977), (5, 978)], 128),
]


@pytest.mark.parametrize("fmt", ["absmax32", "int4"])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("K,shapes,bs", CASES)
def test_grouped_formats_match_oracle(fmt, batch, K, shapes, bs):
    _grouped_case(fmt, batch, K, shapes, bs)


@pytest.mark.parametrize("fmt", ["absmax32", "int4"])
@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("K,shapes,bs", XLDS_CASES)
def test_grouped_formats_several_passes_match_oracle(fmt, batch, K, shapes, bs):
    _grouped_case(fmt, batch, K, shapes, bs)


def _grouped_case(fmt, batch, K, shapes, bs):
    qs, items = [], []
    for N, seed in shapes:
        q, t = _encode(fmt, seed, N, K, bs)
        xb = synth.activations(seed + 50, batch, K)
        base, yv = G.guarded(batch * N, torch.bfloat16)
        items.append((t, N, G.x_to_device(xb), yv.view(batch, N)))
        qs.append((q, N, xb, base, yv))
    print(f"[grouped_{fmt}] K={K} B={batch} bs={bs} N={[n for n, _ in shapes]}", flush=True)
    outs = []
    for dynamic in (True, False):
        for (_, _, _, _, yv) in qs:
            yv.fill_(float("nan"))
        grp = nf4.GemvGroup(items, K, dynamic=dynamic)
        grp.launch()
        torch.cuda.synchronize()
        outs.append([G.bits16(yv).copy() for (_, _, _, _, yv) in qs])
    for a, b in zip(*outs):
        assert np.array_equal(a, b), "dynamic and fixed split differ"
    for (q, N, xb, base, yv) in qs:
        assert G.guards_intact(base, batch * N), "write outside y"
        y = G.bf16_to_f64(G.bits16(yv)).reshape(batch, N)
        yr, bound = _reference(fmt, q, N, K, xb)
        ok, worst = G.gemv_within_tolerance(y, yr, bound)
        assert ok, f"{fmt} grouped N={N} K={K} B={batch}: worst error/bound = {worst:.3g}"


def test_grouped_formats_skip_bad_descriptors():
    """A descriptor with a misaligned scale array is skipped (its y keeps its
    old contents); the others are computed."""
    K = 1024
    q0, t0 = _encode("absmax32", 960, 64, K, 64)
    q1, t1 = _encode("absmax32", 961, 32, K, 64)
    buf = torch.zeros(t1.absmax.numel() + 1, dtype=torch.float32, device=G.dev())
    shifted = buf.view(torch.uint8)[2:2 + 4 * t1.absmax.numel()]  # 2-byte aligned only
    shifted.copy_(t1.absmax.view(torch.uint8))
    xb = synth.activations(962, 1, K)
    x = G.x_to_device(xb)
    y0 = torch.full((1, 64), 5.0, dtype=torch.bfloat16, device=G.dev())
    y1 = torch.full((1, 32), 5.0, dtype=torch.bfloat16, device=G.dev())
    grp = nf4.GemvGroup([(t0, 64, x, y0), (t1, 32, x, y1)], K)
    # point item 1's absmax at the misaligned copy in the uploaded table
    table = grp.table.view(torch.int64).view(-1, 8)
    table[1, 1] = shifted.data_ptr()
    grp.launch()
    torch.cuda.synchronize()
    assert torch.all(y1 == 5.0), "the misaligned matrix was not skipped"
    yr, S = oracle.gemv_sl(q0, 64, K, xb)
    ok, worst = G.gemv_within_tolerance(G.bf16_to_f64(G.bits16(y0)).reshape(1, 64), yr, S)
    assert ok, f"worst error/bound = {worst:.3g}"
