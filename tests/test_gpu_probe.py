"""The bandwidth probes (measurement helpers beside the hot path) do what
include/nf4_probe.h says: the expand copy writes (w, w^1, w^2, w^3) for each
source dword, and the streaming read runs over ragged sizes without touching
anything but its sink."""
import numpy as np
import pytest
import torch

import w4a16_gemv_amd as nf4
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [4, 4096, 1 << 20, (1 << 20) + 12])
def test_expand_copy_pattern(nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=G.dev())
    dst = torch.zeros(4 * nbytes + 64, dtype=torch.uint8, device=G.dev())
    nf4.probe_expand_copy(src, dst)
    torch.cuda.synchronize()
    w = src.cpu().numpy().view(np.uint32)
    got = dst[:4 * nbytes].cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(got, np.stack([w, w ^ 1, w ^ 2, w ^ 3], axis=1))
    assert int(torch.count_nonzero(dst[4 * nbytes:])) == 0, "write past the end"


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 24])
def test_stream_read_runs(nbytes):
    src = torch.zeros(nbytes, dtype=torch.uint8, device=G.dev())
    sink = torch.full((1,), 7, dtype=torch.int32, device=G.dev())
    nf4.probe_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7  # zeros never match the keep-alive pattern
