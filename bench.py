#!/usr/bin/env python3
"""Throughput of the NF4 double-quant dequant and fused W4A16 GEMV on one GPU.

One step = one pass of the whole hot path over the decode-step workload of a
32-layer 7B-shaped model: the 224 batch-1 fused GEMVs of the weight sweep
(per layer 4 x 4096->4096, 2 x 4096->11008, 1 x 11008->4096; 6.48e9 weights,
3.34 GB of NF4 data) plus the standalone dequant of one 8192 x 28672 weight to
bf16.  Inputs are synthetic N(0, 0.02) weights drawn on the GPU and encoded by
the library's own quantizer; they are resident in HBM before timing starts.

Schedules (--schedule):
  stream   (default) the sweep as one grouped launch per K (all 192 K=4096
           GEMVs, then the 32 K=11008 ones): every weight byte streams through
           one persistent grid, as in a weight sweep where the GEMVs are
           independent.
  layered  per layer: q/k/v grouped, o, gate/up grouped, down -- the launch
           order a real decode step with layer dependencies would use.
The step is captured once in a HIP graph and replayed.

The timed steps are launched eagerly on one stream (three launches per step
in the stream schedule), with HIP events bracketing the dominant kernel -- the
K=4096 grouped GEMV, 192 matrices, 2.60 GB per launch -- in every step.  Before
the W warm-up steps, the captured step is replayed for at least --prewarm
seconds: a cold GPU runs this path about 10% slower for its first few hundred
milliseconds of load while its clocks settle.

--workload picks another configuration as a context measurement (the default
`sweep` is the headline): sweep_absmax32 / sweep_int4 (the same sweep and big
dequant in the single-level and INT4 formats, grouped launches of
nf4_gemv_grouped_absmax32 / int4_gemv_grouped; no CPU baseline), dequant_1k /
dequant_4k (1024^2 and 4096^2 bf16 dequant), qwen_b1 (the 7 Qwen2.5-1.5B-shaped GEMVs),
qwen_b1_grouped (the same 7 as 4 launches: q/k/v and gate/up grouped), llama_b1 / llama_b4 /
llama_b8 (the 3 Llama-7B-shaped GEMVs at batch 1, 4, 8; llama_b2 / b3 / b5 / b6 / b7 at
the other batches), llama_b16 / llama_b64
/ llama_b128 (the same 3 matrices times 16, 64, 128 activation rows through
nf4_gemm, the matrix-core product; roofline against the bf16 MFMA peak), and
each of the first six with the suffix _absmax32 for the single-level format (one fp32 absmax per
block: nf4_dequant_absmax32 / nf4_gemv_absmax32, encoded by
nf4_quantize_absmax32) or _int4 for the INT4 asymmetric group format
(int4_dequant / int4_gemv, group 128, encoded by int4_quantize).  These run one
nf4_dequant / nf4_gemv call per matrix over copies of the encoded data rotated
so that every step reads past the 256 MB MALL (cold HBM), timed from HIP
graphs, and report the kernel of their largest matrix as the dominant one.

Reported: value = algorithmic bytes per step / step time (GB/s); roofline of
the dominant kernel = its algorithmic bytes per launch / its average duration
over the timed steps; traffic = its HBM bytes per launch from the committed
rocprofv3 counter summary (profiles/), given only when that summary was taken
on the current kernel source; the CPU oracle timed on a bounded sample of the
same workload.
Algorithmic bytes: dequant ceil(n/2) + ceil(n/64) + 2 ceil(n/16384) + 516 + 2n;
GEMV ceil(NK/2) + ceil(NK/64) + 2 ceil(NK/16384) + 516 + 2KB + 2NB; in the
single-level format 4 ceil(n/64) bytes of scales replace the second-level terms,
in the INT4 format 4 ceil(n/G) bytes of fp16 scales and zero points.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CONTEXT_WORKLOADS = ("dequant_1k", "dequant_4k", "qwen_b1", "llama_b1", "llama_b4", "llama_b8")
# the same Llama-shaped GEMVs at the other batches of the GEMV (nf4 format only)
LLAMA_OTHER_BATCHES = ("llama_b2", "llama_b3", "llama_b5", "llama_b6", "llama_b7")
# the Qwen2.5-1.5B layer in four launches: q/k/v grouped, o, gate/up grouped,
# down (double-quantized format)
GROUPED_WORKLOADS = ("qwen_b1_grouped",)
QWEN_LAUNCHES = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
# batched products on the matrix cores (nf4_gemm), double-quantized format only
GEMM_WORKLOADS = ("llama_b16", "llama_b64", "llama_b128")
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "NF4 dequant & fused GEMV: achieved HBM GB/s and % of MI355X peak (1 GPU)"
# what the path computes in: the GEMV multiplies bf16 activations by each
# weight written exactly as two bf16 terms (hi + lo, within 2^-16 of the fp32
# weight) with fp32 accumulation; the dequant computes in fp32 and rounds once
DTYPE_NOTE = ("GEMV: bf16 x bf16 products (weight as an exact hi + lo bf16 pair; single "
              "launches at batch 3-8 with K <= 4096: exact fp32 weight x widened bf16 activation "
              "in fp32 FMAs), fp32 accumulation, bf16 y; dequant: fp32 arithmetic, RNE to bf16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dequant_bytes(n: int) -> int:
    return (n + 1) // 2 + -(-n // 64) + 2 * -(-n // 16384) + 516 + 2 * n


def gemv_bytes(N: int, K: int, B: int = 1) -> int:
    n = N * K
    return (n + 1) // 2 + -(-n // 64) + 2 * -(-n // 16384) + 516 + 2 * K * B + 2 * N * B



SWEEP_WORKLOADS = ("sweep", "sweep_absmax32", "sweep_int4")


def sweep_format(workload: str) -> str:
    return "double" if workload == "sweep" else workload.split("_", 1)[1]


def format_bytes(fmt: str):
    """(dequant_bytes(n), gemv_bytes(N, K, B)) of a format at the sweep's
    block sizes (64 and 256; INT4 groups of 128)."""
    if fmt == "double":
        return dequant_bytes, gemv_bytes
    g = 64 if fmt == "absmax32" else 128

    def dq(n):
        return (n + 1) // 2 + 4 * -(-n // g) + 2 * n

    def gv(N, K, B=1):
        return (N * K + 1) // 2 + 4 * -(-N * K // g) + 2 * K * B + 2 * N * B
    return dq, gv


def build_workload(dev, fmt: str = "double"):
    """The sweep's 224 matrices and the 8192 x 28672 weight, drawn on the GPU
    and encoded by the library's own quantizer of the format (double: NF4
    double-quantized, bs 64 / s2 256; absmax32: NF4 with one fp32 absmax per
    64-block; int4: INT4 asymmetric, groups of 128)."""
    import torch

    import synth
    import w4a16_gemv_amd as nf4

    t0 = time.time()
    code2 = nf4.nf4_code2_linear().to(dev)
    ws = None

    def encode(w):
        nonlocal ws
        if fmt == "absmax32":
            return nf4.nf4_quantize_absmax32(w, 64)
        if fmt == "int4":
            return nf4.int4_quantize(w, 128)
        need = nf4.load().nf4_quantize_workspace_size(w.numel(), 64)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        return nf4.nf4_quantize(w, 64, 256, code2=code2, workspace=ws)

    # each layer reads its own activations: xs[(layer, slot)], see synth.SWEEP_X_SLOT
    xs = {}
    layers = []
    for L in range(synth.SWEEP_LAYERS):
        mats = []
        for g in synth.sweep_layer(L):
            slot = synth.SWEEP_X_SLOT[g.name.split("_", 1)[1]]
            if (L, slot) not in xs:
                xs[(L, slot)] = synth.activations_device(synth.sweep_x_seed(L, slot), 1, g.K, dev)
            w = synth.weights_device(g.seed, g.N * g.K, dev)
            t = encode(w)
            del w
            y = torch.empty(1, g.N, dtype=torch.bfloat16, device=dev)
            mats.append((g, t, y, xs[(L, slot)]))
        layers.append(mats)
    big = synth.DEQUANT_BIG
    wb = synth.weights_device(big.seed, big.n, dev)
    tb = encode(wb)
    del wb, ws
    out = torch.empty(big.n, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] workload ({fmt}) encoded on the GPU in {time.time() - t0:.1f} s")
    return dict(layers=layers, xs=xs, big=(big, tb, out), code2=code2, fmt=fmt)


DOMINANT_K = 4096
DOMINANT_KERNEL = ("gemv_wave_kernel<1, 2, 1, 4, true, 0, true> (nf4_gemv_grouped, K=4096, "
                   "192 matrices)")
DOMINANT_KERNEL_FMT = {
    "absmax32": "gemv_wave_kernel<1, 2, 1, 4, true, 1, true> (nf4_gemv_grouped_absmax32, K=4096, "
                "192 matrices)",
    "int4": "gemv_wave_kernel<1, 2, 1, 4, true, 2, true> (int4_gemv_grouped, K=4096, 192 matrices)",
}
KERNEL_SOURCE = os.path.join(ROOT, "w4a16_gemv_amd", "csrc", "nf4_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_wave_k4096_sweep_traffic.txt")


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none or it was taken on other kernel
    source.  The file holds `key: value` lines (see its header)."""
    try:
        kv = {}
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != source_digest():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def make_step(wl, schedule):
    """Returns (gemv_fns, dequant_fn, gemv_launches)."""
    import w4a16_gemv_amd as nf4
    groups = []
    if schedule == "stream":
        for K in (4096, 11008):
            items = [(t, g.N, x, y) for mats in wl["layers"] for (g, t, y, x) in mats
                     if g.K == K]
            groups.append(nf4.GemvGroup(items, K))
    else:
        for mats in wl["layers"]:
            q, k, v, o, gate, up, down = mats
            for sel in ((q, k, v), (o,), (gate, up), (down,)):
                K = sel[0][0].K
                groups.append(nf4.GemvGroup([(t, g.N, x, y) for (g, t, y, x) in sel], K))
    big, tb, out = wl["big"]

    def gemvs():
        for grp in groups:
            grp.launch()

    def dequant():
        tb.dequant(out=out)

    gemvs.groups = groups
    return gemvs, dequant, len(groups)


def capture(fn, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()          # eager run on the capture stream first
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, warmup, stream):
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps  # ms


MALL_BYTES = 256 << 20
VALU_PEAK_TFLOPS = 157.3


def build_context(dev, name, bs=None):
    """One of the smaller configurations, encoded once and copied into enough
    sets that one pass over all sets reads more than twice the MALL.
    Returns dict(sets, step_bytes, flops, launches, dominant, run)."""
    import torch

    import synth
    import w4a16_gemv_amd as nf4
    code2 = nf4.nf4_code2_linear().to(dev)
    single = name.endswith("_absmax32")        # the single-level format
    int4 = name.endswith("_int4")              # the INT4 asymmetric group format
    base_name = name.rsplit("_", 1)[0] if (single or int4) else name
    if bs is None:
        bs = 128 if int4 else 64
    if int4:
        def dq_bytes(n):
            return (n + 1) // 2 + 4 * -(-n // bs) + 2 * n

        def gv_bytes(N, K, B):
            return (N * K + 1) // 2 + 4 * -(-N * K // bs) + 2 * K * B + 2 * N * B
    elif single:
        def dq_bytes(n):
            return (n + 1) // 2 + 4 * -(-n // bs) + 2 * n

        def gv_bytes(N, K, B):
            return (N * K + 1) // 2 + 4 * -(-N * K // bs) + 2 * K * B + 2 * N * B
    else:
        def dq_bytes(n):
            return (n + 1) // 2 + -(-n // bs) + 2 * -(-n // (bs * 256)) + 516 + 2 * n

        def gv_bytes(N, K, B):
            n = N * K
            return (n + 1) // 2 + -(-n // bs) + 2 * -(-n // (bs * 256)) + 516 + 2 * K * B + 2 * N * B

    def encode(seed, n, outliers=False):
        w = synth.weights_device(seed, n, dev, outliers=outliers)
        if int4:
            t = nf4.int4_quantize(w, bs)
        elif single:
            t = nf4.nf4_quantize_absmax32(w, bs)
        else:
            ws = torch.empty(nf4.load().nf4_quantize_workspace_size(n, bs), dtype=torch.uint8,
                             device=dev)
            t = nf4.nf4_quantize(w, bs, 256, code2=code2, workspace=ws)
            del ws
        del w
        return t

    def clone(t):
        if int4:
            return nf4.Int4Tensor(t.packed.clone(), t.scales.clone(), t.zeros.clone(), t.n,
                                  t.group_size)
        if single:
            return nf4.NF4Absmax32Tensor(t.packed.clone(), t.absmax.clone(), t.n, t.blocksize)
        return nf4.NF4Tensor(t.packed.clone(), t.absmax_q.clone(), t.absmax2.clone(), t.code2,
                             t.offset, t.n, t.blocksize, t.s2_blocksize)

    if base_name.startswith("dequant"):
        cfg = synth.DEQUANT_1K if base_name == "dequant_1k" else synth.DEQUANT_4K
        base = encode(cfg.seed, cfg.n, cfg.outliers)
        set_bytes = dq_bytes(cfg.n)
        nsets = max(2, -(-2 * MALL_BYTES // set_bytes))
        sets = []
        for _ in range(nsets):
            sets.append((clone(base), torch.empty(cfg.n, dtype=torch.bfloat16, device=dev)))

        def run(st, dominant_only=False):
            t, out = st
            t.dequant(out=out)
        return dict(sets=sets, step_bytes=set_bytes, flops=0, launches=1, run=run, blocksize=bs,
                    copy_read_bytes=set_bytes - 2 * cfg.n,
                    dominant=f"dequant_vec_kernel ({cfg.rows}x{cfg.cols}"
                             f"{', fp32 absmax' if single else ''}{', int4' if int4 else ''})",
                    dominant_bytes=set_bytes, dominant_flops=0)

    if name == "qwen_b1_grouped":
        gemvs, batch = synth.QWEN_GEMVS, 1
        xs = {K: synth.activations_device(synth.QWEN_X_SEED, 1, K, dev)
              for K in {g.K for g in gemvs}}
        base = {g.name.split("_")[1]: (g, encode(g.seed, g.N * g.K)) for g in gemvs}
        set_bytes = sum(gv_bytes(g.N, g.K, 1) for g in gemvs)
        nsets = max(2, -(-2 * MALL_BYTES // set_bytes))
        sets = []
        for _ in range(nsets):
            launches = []
            for sel in QWEN_LAUNCHES:
                items = []
                for nm in sel:
                    g, t = base[nm]
                    items.append((clone(t), g.N, xs[g.K],
                                  torch.empty(1, g.N, dtype=torch.bfloat16, device=dev)))
                launches.append(nf4.GemvGroup(items, items[0][0].n // items[0][1]))
            sets.append(launches)
        dom = 2   # gate/up, the largest launch
        dom_rows = sum(base[nm][0].N for nm in QWEN_LAUNCHES[dom])
        K_dom = base["gate"][0].K

        def run(st, dominant_only=False):
            for i, grp in enumerate(st):
                if not dominant_only or i == dom:
                    grp.launch()
        return dict(sets=sets, step_bytes=set_bytes, flops=sum(2 * g.N * g.K for g in gemvs),
                    launches=len(QWEN_LAUNCHES), run=run, batch=1, blocksize=bs,
                    dominant=f"nf4_gemv_grouped gate+up {dom_rows}x{K_dom} batch 1",
                    dominant_bytes=sum(gv_bytes(base[nm][0].N, K_dom, 1)
                                       for nm in QWEN_LAUNCHES[dom]),
                    dominant_flops=2 * dom_rows * K_dom)

    if base_name == "qwen_b1":
        gemvs, batch, xseed = synth.QWEN_GEMVS, 1, synth.QWEN_X_SEED
    else:
        batch = int(base_name.split("_b")[1])
        gemvs, xseed = synth.LLAMA_GEMVS, synth.llama_x_seed(batch)
    xs = {K: synth.activations_device(xseed, batch, K, dev) for K in {g.K for g in gemvs}}
    base = [(g, encode(g.seed, g.N * g.K)) for g in gemvs]
    set_bytes = sum(gv_bytes(g.N, g.K, batch) for g in gemvs)
    nsets = max(2, -(-2 * MALL_BYTES // set_bytes))
    sets = []
    for _ in range(nsets):
        sets.append([(g, clone(t), torch.empty(batch, g.N, dtype=torch.bfloat16, device=dev))
                     for g, t in base])
    dom = max(range(len(gemvs)), key=lambda i: gemvs[i].N * gemvs[i].K)
    gd = gemvs[dom]

    gemm = batch > 8
    ws = None
    if gemm:
        # one split-K scratch workspace for all the products (serial on one stream)
        need = max(nf4.load().nf4_gemm_workspace_size(batch, g.N, g.K) for g in gemvs)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def run(st, dominant_only=False):
        for i, (g, t, y) in enumerate(st):
            if not dominant_only or i == dom:
                if gemm:
                    t.gemm(g.N, g.K, xs[g.K], y, workspace=ws)
                else:
                    t.gemv(g.N, g.K, xs[g.K], y)
    kname = ("nf4_gemm" if gemm else "int4_gemv" if int4 else
             "nf4_gemv_absmax32" if single else "nf4_gemv")
    return dict(sets=sets, step_bytes=set_bytes, flops=sum(2 * g.N * g.K * batch for g in gemvs),
                launches=len(gemvs), run=run, batch=batch, blocksize=bs, gemm=gemm,
                dominant=f"{kname} {gd.N}x{gd.K} batch {batch}",
                dominant_bytes=gv_bytes(gd.N, gd.K, batch), dominant_flops=2 * gd.N * gd.K * batch)


def bench_context(args, dev):
    """Small kernels are timed from HIP graphs (eager launches from Python
    cannot keep the GPU busy at 5-20 us per kernel): one graph holds one step
    over every rotating set, a second one only the dominant kernel's launches
    over every set.  Per step / per launch = graph time / number of sets."""
    import torch
    wl = build_context(dev, args.workload, args.blocksize)
    args.blocksize = wl["blocksize"]
    sets = wl["sets"]
    stream = torch.cuda.Stream(dev)

    def all_steps():
        for st in sets:
            wl["run"](st)

    def all_dominant():
        for st in sets:
            wl["run"](st, dominant_only=True)

    g_steps = capture(all_steps, stream)
    g_dom = capture(all_dominant, stream)
    t0 = time.time()
    with torch.cuda.stream(stream):
        while time.time() - t0 < args.prewarm:
            g_steps.replay()
            torch.cuda.synchronize()
    reps = max(1, -(-args.steps // len(sets)))      # at least args.steps steps
    ms = time_graph(g_steps, reps, args.warmup, stream) / len(sets)
    dom_us = 1e3 * time_graph(g_dom, reps, args.warmup, stream) / len(sets)
    value = wl["step_bytes"] / (ms * 1e-3) / 1e9
    dom_gbs = wl["dominant_bytes"] / (dom_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": wl["dominant"], "achieved": round(dom_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": None, "bytes_per_launch": wl["dominant_bytes"], "avg_launch_us": round(dom_us, 3)}
    if wl.get("gemm"):
        # a contraction on the matrix cores: useful flops 2 M N K against the
        # dense bf16 MFMA peak (the exact hi + lo weight split issues twice that)
        tf = wl["dominant_flops"] / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": wl["dominant"], "achieved": round(tf, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": wl["dominant_flops"], "avg_launch_us": round(dom_us, 3),
                "hbm": {"achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                        "bytes_per_launch": wl["dominant_bytes"]}}
    elif wl["dominant_flops"]:
        tf = wl["dominant_flops"] / (dom_us * 1e-6) / 1e12
        roof["alu"] = {"achieved_tflops": round(tf, 2), "peak_tflops": VALU_PEAK_TFLOPS,
                       "frac": round(tf / VALU_PEAK_TFLOPS, 4)}
    log(f"[bench] {args.workload}: step {ms * 1e3:.1f} us ({value:.0f} GB/s); dominant "
        f"{dom_us:.1f} us ({dom_gbs:.0f} GB/s); {len(sets)} rotating sets, {reps} graph replays")
    ceiling = None
    if wl.get("copy_read_bytes") and not args.no_ceiling:
        # the same stream without the decode, at the same size and rotation:
        # read R bytes, write 4 R with streaming stores (nf4_probe_expand_copy)
        import w4a16_gemv_amd as nf4
        rb = wl["copy_read_bytes"] // 16 * 16
        pairs = [(torch.full((rb,), 7, dtype=torch.uint8, device=dev),
                  torch.empty(4 * rb, dtype=torch.uint8, device=dev)) for _ in sets]

        def all_copies():
            for src, dst in pairs:
                nf4.probe_expand_copy(src, dst)
        g_copy = capture(all_copies, stream)
        copy_us = 1e3 * time_graph(g_copy, reps, args.warmup, stream) / len(sets)
        ceiling = {"expand_copy_1to4": {"bytes": 5 * rb, "us": round(copy_us, 3),
                                        "gbs": round(5 * rb / (copy_us * 1e-6) / 1e9, 1)}}
        roof["frac_of_copy_ceiling"] = round(dom_gbs / ceiling["expand_copy_1to4"]["gbs"], 4)
        log(f"[bench] ceiling: 1:4 expand copy of {5 * rb} bytes {copy_us:.2f} us "
            f"({ceiling['expand_copy_1to4']['gbs']:.0f} GB/s); dequant at "
            f"{roof['frac_of_copy_ceiling']:.3f} of its rate")
        del pairs
    return dict(value=value, ms=ms, roofline=roof, sets=len(sets), launches=wl["launches"], ceiling=ceiling,
                step_bytes=wl["step_bytes"], batch=wl.get("batch", 1), steps=reps * len(sets),
                step_tflops=wl["flops"] / (ms * 1e-3) / 1e12 if wl["flops"] else None)


def dequant_4k_context(dev, reps: int, warmup: int):
    """The 4096 x 4096 dequant (config 2: with outliers, bs 64 / s2 256) as a
    single launch per call, bf16 and fp16 outputs, timed from HIP graphs over
    enough copies of the data to read past the MALL (cold HBM), beside three
    plain streams of the same size on the same rotation: the library's 1 : 4
    expand copy probe (read R, write 4 R with streaming stores), torch's
    elementwise uint8 -> int32 cast (the same R in, 4 R out; an independent
    kernel), and a device-to-device memcpy (torch copy_) of the same total
    bytes; and the bf16 dequant on one set of buffers, which stay in the MALL
    (cache-resident, labelled so).  Returns per-launch microseconds and GB/s
    of each."""
    import torch

    import synth
    import w4a16_gemv_amd as nf4
    cfg = synth.DEQUANT_4K
    n = cfg.n
    code2 = nf4.nf4_code2_linear().to(dev)
    w = synth.weights_device(cfg.seed, n, dev, outliers=cfg.outliers)
    ws = torch.empty(nf4.load().nf4_quantize_workspace_size(n, 64), dtype=torch.uint8,
                     device=dev)
    base = nf4.nf4_quantize(w, 64, 256, code2=code2, workspace=ws)
    del w, ws
    nbytes = dequant_bytes(n)
    nsets = max(2, -(-2 * MALL_BYTES // nbytes))
    sets = [nf4.NF4Tensor(base.packed.clone(), base.absmax_q.clone(), base.absmax2.clone(),
                          code2, base.offset, n) for _ in range(nsets)]
    outs = {dt: [torch.empty(n, dtype=dt, device=dev) for _ in range(nsets)]
            for dt in (torch.bfloat16, torch.float16)}
    rb = (n // 2) // 16 * 16                          # the packed bytes (read side)
    src = [torch.full((rb,), 7, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    dst = [torch.empty(4 * rb, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    dst32 = [torch.empty(rb, dtype=torch.int32, device=dev) for _ in range(nsets)]
    half = nbytes // 2 // 16 * 16                     # memcpy: read half, write half
    msrc = [torch.full((half,), 3, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    mdst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    stream = torch.cuda.Stream(dev)
    runs = {
        "dequant_bf16": (lambda: [t.dequant(out=o) for t, o in zip(sets, outs[torch.bfloat16])],
                         nbytes),
        "dequant_fp16": (lambda: [t.dequant(out=o) for t, o in zip(sets, outs[torch.float16])],
                         nbytes),
        "expand_copy_1to4": (lambda: [nf4.probe_expand_copy(a, b) for a, b in zip(src, dst)],
                             5 * rb),
        "torch_cast_u8_to_i32": (lambda: [b.copy_(a) for a, b in zip(src, dst32)], 5 * rb),
        "memcpy_d2d": (lambda: [b.copy_(a) for a, b in zip(msrc, mdst)], 2 * half),
        # the same input and output every launch: 42 MB stay in the 256 MB
        # MALL, so this one is cache-resident (not an HBM figure)
        "dequant_bf16_cache_resident": (
            lambda: [sets[0].dequant(out=outs[torch.bfloat16][0]) for _ in range(nsets)], nbytes),
    }
    res = {}
    for name, (fn, nb) in runs.items():
        g = capture(fn, stream)
        us = 1e3 * time_graph(g, max(1, reps // nsets), warmup, stream) / nsets
        res[name] = {"us": round(us, 3), "bytes": nb, "gbs": round(nb / (us * 1e-6) / 1e9, 1)}
        del g
    res["rotating_sets"] = nsets
    res["dequant_bf16"]["frac"] = round(res["dequant_bf16"]["gbs"] / HBM_PEAK_GBS, 4)
    res["dequant_fp16"]["frac"] = round(res["dequant_fp16"]["gbs"] / HBM_PEAK_GBS, 4)
    log(f"[bench] dequant 4096^2: bf16 {res['dequant_bf16']['us']:.2f} us, fp16 "
        f"{res['dequant_fp16']['us']:.2f} us; same-size streams: expand copy "
        f"{res['expand_copy_1to4']['us']:.2f} us, torch u8->i32 cast "
        f"{res['torch_cast_u8_to_i32']['us']:.2f} us, memcpy {res['memcpy_d2d']['us']:.2f} us; "
        f"bf16 cache-resident (same buffers) {res['dequant_bf16_cache_resident']['us']:.2f} us")
    return res


def cpu_info():
    """Host description for the CPU baseline: logical CPUs (and those this
    process may run on) and the model name from /proc/cpuinfo."""
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def gemv_outputs_ok(y_gpu_bits, y_ref, S):
    """The GEMV acceptance rule (as in the tests): each bf16 output must be the
    round-to-nearest-even bf16 of some real within 2^-14 S of the fp64 oracle
    value.  Returns (ok, number of outputs outside)."""
    import numpy as np
    import torch

    def bf16(v):
        return torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(torch.bfloat16) \
            .to(torch.float64).numpy()
    y = (y_gpu_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lo, hi = bf16(y_ref - 2.0 ** -14 * S), bf16(y_ref + 2.0 ** -14 * S)
    bad = int(np.count_nonzero(~((y >= lo) & (y <= hi))))
    return bad == 0, bad


def cpu_baseline(wl, seconds: float):
    """The oracle (plain C, OpenMP over outputs) timed on the host cores on a
    bounded sample of the same workload: the sweep's GEMVs in order, then a
    slice of the big dequant, until about `seconds` of wall time is spent,
    with all threads; then a smaller sample on one thread.  Every GEMV the
    oracle computes is also checked against the GPU's output of the last
    timed step (the acceptance rule of the tests)."""
    import numpy as np
    import torch

    import oracle
    threads = oracle.max_threads()

    def host_q(t, n=None):
        n = t.n if n is None else n
        return oracle.Quantized(t.packed[: (n + 1) // 2].cpu().numpy(),
                                t.absmax_q[: -(-n // 64)].cpu().numpy(),
                                t.absmax2[: -(-n // 16384)].cpu().numpy().view(np.uint16),
                                t.code2.cpu().numpy().view(np.uint16), t.offset, n)

    def run(budget_s, max_gemvs, n_dq, check):
        done_bytes, elems, elapsed, ngemv, checked, bad = 0, 0, 0.0, 0, 0, 0
        for mats in wl["layers"]:
            for (g, t, y, x) in mats:
                if ngemv >= max_gemvs or elapsed >= budget_s:
                    break
                q = host_q(t)
                xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
                s0 = time.perf_counter()
                yr, S = oracle.gemv(q, g.N, g.K, xb)
                elapsed += time.perf_counter() - s0
                done_bytes += gemv_bytes(g.N, g.K)
                elems += g.N * g.K
                ngemv += 1
                if check:
                    ok, nbad = gemv_outputs_ok(
                        y.view(torch.int16).cpu().numpy().view(np.uint16), yr, S)
                    checked += 1
                    bad += nbad
        big, tb, _ = wl["big"]
        n_slice = min(big.n, n_dq)
        q = host_q(tb, n_slice)
        s0 = time.perf_counter()
        oracle.dequant(q)
        elapsed += time.perf_counter() - s0
        done_bytes += dequant_bytes(n_slice)
        elems += n_slice
        return dict(bytes=done_bytes, elems=elems, s=elapsed, ngemv=ngemv, n_dq=n_slice,
                    checked=checked, bad=bad)

    full = run(0.8 * seconds, 224, 1 << 24, check=True)
    oracle.set_threads(1)
    try:
        one = run(0.15 * seconds, 8, 1 << 22, check=False)
    finally:
        oracle.set_threads(threads)
    return {"value": round(full["bytes"] / full["s"] / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "elements_per_s": round(full["elems"] / full["s"], 1),
            "sample": f"first {full['ngemv']} of the 224 sweep GEMVs (fp64 oracle GEMV, all "
                      f"rows) + the first {full['n_dq']} elements of the 8192x28672 dequant; "
                      f"{full['s']:.1f} s of wall time",
            "gemv_outputs_checked": {"gemvs": full["checked"],
                                     "outputs_outside_tolerance": full["bad"]},
            "single_thread": {"value": round(one["bytes"] / one["s"] / 1e9, 4), "unit": "GB/s",
                              "elements_per_s": round(one["elems"] / one["s"], 1), "cores": 1,
                              "sample": f"first {one['ngemv']} sweep GEMVs + the first "
                                        f"{one['n_dq']} dequant elements; {one['s']:.1f} s"},
            **cpu_info()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--schedule", choices=("stream", "layered"), default="stream")
    ap.add_argument("--workload", default="sweep",
                    choices=SWEEP_WORKLOADS + CONTEXT_WORKLOADS + LLAMA_OTHER_BATCHES + GEMM_WORKLOADS
                    + GROUPED_WORKLOADS
                    + tuple(w + "_absmax32" for w in CONTEXT_WORKLOADS)
                    + tuple(w + "_int4" for w in CONTEXT_WORKLOADS))
    ap.add_argument("--blocksize", type=int, default=None,
                    help="block (group) size of the context workloads: default 64, 128 for the "
                         "_int4 workloads (the sweep always uses 64)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--prewarm", type=float, default=1.0,
                    help="seconds of untimed steps before the W warm-up steps")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context timings (all GEMVs, dequant, other schedule)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed steps, run an elementwise copy of exactly 1 GiB "
                         "(1 GiB read, 1 GiB written): the reference for scaling the HBM "
                         "byte counters of a profiler run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the bandwidth probes (plain streaming read of the dominant "
                         "launch's bytes; the dequant's 1:4 read:write stream)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the NF4 dequant / GEMV path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a16_gemv_amd as nf4
    nf4.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload not in SWEEP_WORKLOADS:
        r = bench_context(args, dev)
        print(json.dumps({
            "metric": METRIC, "value": round(r["value"], 1), "unit": "GB/s", "n_gpus": 1,
            "steps": r["steps"], "warmup": args.warmup, "ms_per_step": round(r["ms"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "dtype_note": DTYPE_NOTE,
            "data": "synthetic",
            "config": {"workload": args.workload, "batch": r["batch"], "blocksize": args.blocksize,
                       "s2_blocksize": None if args.workload.endswith(("_absmax32", "_int4"))
                       else 256,
                       "launches_per_step": r["launches"],
                       "bytes_per_step": r["step_bytes"], "rotating_sets": r["sets"],
                       "prewarm_s": args.prewarm},
            "pct_of_peak": round(100 * r["value"] / HBM_PEAK_GBS, 2),
            "step_tflops": None if r["step_tflops"] is None else round(r["step_tflops"], 2),
            "roofline": r["roofline"], "ceiling": r["ceiling"], "cpu_baseline": None}), flush=True)
        return
    fmt = sweep_format(args.workload)
    dq_bytes_f, gv_bytes_f = format_bytes(fmt)
    wl = build_workload(dev, fmt)
    stream = torch.cuda.Stream(dev)

    # A captured graph keeps device pointers only: the groups (descriptor
    # tables, scheduling workspaces) it launches must outlive it, so each
    # graph is stored with the step functions that own them.
    per_step = {}
    for sched in ("stream", "layered"):
        gemvs, dequant, nlaunch = make_step(wl, sched)
        g_step = capture(lambda: (gemvs(), dequant()), stream)
        g_gemv = capture(gemvs, stream)
        per_step[sched] = dict(graph=g_step, gemv_graph=g_gemv, launches=nlaunch,
                               owners=(gemvs, dequant))
    dq_owner = make_step(wl, "stream")
    g_dq = capture(dq_owner[1], stream)

    n_gemv_bytes = sum(gv_bytes_f(g.N, g.K) for mats in wl["layers"] for (g, *_) in mats)
    big = wl["big"][0]
    n_dq_bytes = dq_bytes_f(big.n)
    step_bytes = n_gemv_bytes + n_dq_bytes

    # pre-warm (clocks to steady state), then W warm-up steps
    t0 = time.time()
    with torch.cuda.stream(stream):
        while time.time() - t0 < args.prewarm:
            per_step[args.schedule]["graph"].replay()
            torch.cuda.synchronize()
    gemvs, dequant, launches = make_step(wl, args.schedule)
    dom = [g for g in gemvs.groups if g.K == DOMINANT_K] if args.schedule == "stream" else []
    dom_bytes = sum(gv_bytes_f(it[1], DOMINANT_K) for it in dom[0].items) if dom else 0

    def step(ev=None):
        for grp in gemvs.groups:
            if ev is not None and dom and grp is dom[0]:
                ev[0].record(stream)
                grp.launch()
                ev[1].record(stream)
            else:
                grp.launch()
        dequant()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # timed region: exactly args.steps steps, events around the dominant kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            step(evs[i])
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms * 1e-3) / 1e9
    dom_us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / args.steps if dom else None

    ceiling = None
    if not args.no_ceiling:
        # the hot path's memory streams without its arithmetic (bandwidth
        # probes in libnf4): a plain streaming read of the dominant launch's
        # bytes, and the dequant's 1 : 4 read : write stream
        rd = torch.empty((dom_bytes + 15) // 16 * 16 if dom else 1 << 30, dtype=torch.uint8,
                         device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        src = torch.empty((big.n + 1) // 2 // 4 * 4, dtype=torch.uint8, device=dev)
        dst = torch.empty(4 * src.numel(), dtype=torch.uint8, device=dev)

        def timed(fn, reps=5):
            with torch.cuda.stream(stream):
                fn()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    fn()
                b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps * 1e-3  # s

        t_rd = timed(lambda: nf4.probe_stream_read(rd, sink))
        t_cp = timed(lambda: nf4.probe_expand_copy(src, dst))
        ceiling = {"stream_read": {"bytes": rd.numel(), "gbs": round(rd.numel() / t_rd / 1e9, 1)},
                   "expand_copy_1to4": {"bytes": 5 * src.numel(),
                                        "gbs": round(5 * src.numel() / t_cp / 1e9, 1)}}
        log(f"[bench] ceilings: streaming read {ceiling['stream_read']['gbs']:.0f} GB/s, "
            f"1:4 expand copy {ceiling['expand_copy_1to4']['gbs']:.0f} GB/s")
        del rd, src, dst

    if args.calibration_copy:
        src = torch.full((1 << 30,), 0x5A, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # context (not the metric): all GEMVs, the dequant and the other schedule,
    # each replayed as a captured graph
    other = "layered" if args.schedule == "stream" else "stream"
    if args.no_context:
        gemv_ms = dq_ms = other_ms = float("nan")
    else:
        reps = max(10, args.steps)
        gemv_ms = time_graph(per_step[args.schedule]["gemv_graph"], reps, 3, stream)
        dq_ms = time_graph(g_dq, reps, 3, stream)
        other_ms = time_graph(per_step[other]["graph"], reps, 3, stream)
    gemv_gbs = n_gemv_bytes / (gemv_ms * 1e-3) / 1e9
    dq_gbs = n_dq_bytes / (dq_ms * 1e-3) / 1e9
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9 if dom else None
    log(f"[bench] step {ms:.3f} ms ({value:.0f} GB/s); dominant kernel {dom_us or 0:.1f} us "
        f"({dom_gbs or 0:.0f} GB/s); all GEMVs {gemv_ms:.3f} ms ({gemv_gbs:.0f} GB/s, "
        f"{launches} launches); dequant {dq_ms * 1e3:.1f} us ({dq_gbs:.0f} GB/s); "
        f"{other} schedule step {other_ms:.3f} ms")

    dq4k = None
    if not args.no_context and fmt == "double":
        dq4k = dequant_4k_context(dev, max(200, args.steps), 20)

    cpu = None
    if not args.no_cpu_baseline and fmt == "double":
        cpu = cpu_baseline(wl, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu}")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_note": DTYPE_NOTE,
        "data": "synthetic",
        "config": {
            "workload": "decode_sweep_7b_32layers_224gemv_b1+dequant_8192x28672"
                        + ("" if fmt == "double" else "_" + fmt),
            "gemv_weights": sum(g.N * g.K for mats in wl["layers"] for (g, *_) in mats),
            "batch": 1, "blocksize": 128 if fmt == "int4" else 64,
            "s2_blocksize": 256 if fmt == "double" else None,
            "dequant_elems": big.n, "dequant_out": "bf16",
            "schedule": args.schedule, "gemv_launches_per_step": launches,
            "bytes_per_step": step_bytes, "prewarm_s": args.prewarm,
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": None if not dom else {
            "bound": "hbm",
            "kernel": DOMINANT_KERNEL if fmt == "double" else DOMINANT_KERNEL_FMT[fmt],
            "achieved": round(dom_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic() if fmt == "double" else None,
            "bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 3),
            "kernel_source_sha256_16": source_digest(),
            "frac_of_read_ceiling": None if ceiling is None else
            round(dom_gbs / ceiling["stream_read"]["gbs"], 4),
        },
        "all_gemvs": None if args.no_context else {"gbs": round(gemv_gbs, 1), "ms": round(gemv_ms, 4),
                                                   "launches": launches},
        "dequant": None if args.no_context else {
            "kernel": f"dequant_vec_kernel<0, 4, {('double', 'absmax32', 'int4').index(fmt)}> "
                      f"(bf16, 4 steps per lane)", "gbs": round(dq_gbs, 1),
            "us": round(dq_ms * 1e3, 2), "frac": round(dq_gbs / HBM_PEAK_GBS, 4),
            "frac_of_copy_ceiling": None if ceiling is None else
            round(dq_gbs / ceiling["expand_copy_1to4"]["gbs"], 4)},
        "ceiling": ceiling,
        "dequant_4096x4096": dq4k,
        f"{other}_schedule": None if args.no_context else {
            "ms_per_step": round(other_ms, 4),
            "value": round(step_bytes / (other_ms * 1e-3) / 1e9, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
