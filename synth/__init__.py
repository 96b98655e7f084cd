"""Seeded synthetic inputs for the NF4 W4A16 workloads.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no arithmetic of the method: it only draws random weights and
activations and names the workload shapes.  Quantization (turning weights into
the packed NF4 format) is done by the oracle on the CPU side and by the
library's own quantizer on the GPU side.

Workloads (shapes follow the pages: the k/v, q/o and MLP projections of
Qwen2.5-1.5B from "RTX 4060 上的 LLM 量化实测", section "为什么是 k/v projection";
7B-sized layers from "量化与 GEMV", section "为什么 decode 需要量化"; the
4096 x 4096 dequant from the NF4 report's §5):

  dequant_1k   : 1024 x 1024 weight, N(0, 0.02), bf16 output
  dequant_4k   : 4096 x 4096 weight, N(0, 0.02) with 0.1 % of entries x10
  qwen_gemv    : batch-1 GEMVs K=1536 -> N in {1536, 256, 8960}, K=8960 -> 1536
  llama_gemv   : 4096 -> 4096, 4096 -> 11008, 11008 -> 4096 at batch 1, 4, 8
  decode_sweep : 32 layers x [4 x (4096 -> 4096), 2 x (4096 -> 11008),
                 1 x (11008 -> 4096)] batch-1 GEMVs + an 8192 x 28672 dequant

A GEMV "K -> N" has weight W of shape [N][K] (row-major, flattened for the
block/group index) and activations x of shape [B][K].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_FRACTION = 1.0 / 1000.0
OUTLIER_SCALE = 10.0


def weights(seed: int, n: int, outliers: bool = False) -> np.ndarray:
    """n fp32 weights ~ N(0, 0.02) from numpy PCG64(seed); with `outliers`,
    n // 1000 distinct entries (chosen by the same generator) are scaled x10."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(n, dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    if outliers:
        idx = rng.choice(n, n // 1000, replace=False)
        w[idx] *= np.float32(OUTLIER_SCALE)
    return w


def activations_f32(seed: int, batch: int, k: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, k), dtype=np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 data (torch's CPU round-to-nearest-even cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(seed: int, batch: int, k: int) -> np.ndarray:
    """bf16 activations x[batch][k] ~ N(0, 1), as uint16 bit patterns."""
    return to_bf16_bits(activations_f32(seed, batch, k))


# ---- GPU-side draws (benchmark inputs; torch's Philox generator on device) ----

def weights_device(seed: int, n: int, device, outliers: bool = False):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    w.mul_(WEIGHT_STD)
    if outliers:
        idx = torch.randperm(n, generator=g, device=device)[: n // 1000]
        w[idx] *= OUTLIER_SCALE
    return w


def activations_device(seed: int, batch: int, k: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(batch, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


# ---- workload shapes and seeds ----

@dataclass(frozen=True)
class Gemv:
    name: str
    N: int          # output features (rows of W)
    K: int          # input features
    seed: int


@dataclass(frozen=True)
class Dequant:
    name: str
    rows: int
    cols: int
    seed: int
    outliers: bool = False

    @property
    def n(self) -> int:
        return self.rows * self.cols


DEQUANT_1K = Dequant("dequant_1024x1024", 1024, 1024, seed=1)
DEQUANT_4K = Dequant("dequant_4096x4096_outliers", 4096, 4096, seed=2, outliers=True)
DEQUANT_BIG = Dequant("dequant_8192x28672", 8192, 28672, seed=5900)

QWEN_GEMVS = [
    Gemv("qwen_q_1536to1536", 1536, 1536, 300),
    Gemv("qwen_k_1536to256", 256, 1536, 301),
    Gemv("qwen_v_1536to256", 256, 1536, 302),
    Gemv("qwen_o_1536to1536", 1536, 1536, 303),
    Gemv("qwen_gate_1536to8960", 8960, 1536, 304),
    Gemv("qwen_up_1536to8960", 8960, 1536, 305),
    Gemv("qwen_down_8960to1536", 1536, 8960, 306),
]
QWEN_X_SEED = 399

LLAMA_GEMVS = [
    Gemv("llama_4096to4096", 4096, 4096, 400),
    Gemv("llama_4096to11008", 11008, 4096, 401),
    Gemv("llama_11008to4096", 4096, 11008, 402),
]
LLAMA_BATCHES = (1, 4, 8)


def llama_x_seed(batch: int) -> int:
    return 450 + batch


SWEEP_LAYERS = 32
SWEEP_X_SEED = 5999

# Which activation vector of its layer each sweep GEMV reads: q, k and v read
# the attention input, o the attention output, gate and up the MLP input,
# down the MLP's inner activation (K = 11008).
SWEEP_X_SLOT = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}


def sweep_x_seed(layer: int, slot: int) -> int:
    """Seed of activation vector `slot` (0..3) of sweep layer `layer`."""
    return SWEEP_X_SEED + 4 * layer + slot


def sweep_layer(layer: int) -> list[Gemv]:
    """The 7 GEMVs of one 7B-shaped decoder layer (q, k, v, o, gate, up, down)."""
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    return [Gemv(f"L{layer}_{nm}", N, K, 5000 + 10 * layer + j)
            for j, (nm, (N, K)) in enumerate(zip(names, shapes))]


def sweep() -> list[Gemv]:
    out = []
    for layer in range(SWEEP_LAYERS):
        out.extend(sweep_layer(layer))
    return out
