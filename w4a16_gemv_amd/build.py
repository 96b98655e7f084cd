"""Build libnf4.so (the gfx950 HIP library) in-tree with hipcc.

Flags:
  --offload-arch=gfx950     CDNA4 only; no other targets, no host fallback.
  -ffp-contract=off         the dequant formula rounds each product and sum to
                            fp32 on its own; GEMV code uses explicit fmaf.
  -target-feature -packed-fp32-ops
                            no packed fp32 VALU instructions.
The compiler's kernel-resource-usage remarks are parsed into
kernel_resources.txt (registers, scratch, occupancy, LDS per kernel); the
build fails when an instance on the measured hot path (NO_SPILL) spills.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f)
        for f in ("nf4_kernels.hip", "nf4_gemm.hip", "nf4_quantize.hip", "nf4_probe.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnf4.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the scheduling claims are single-lane atomics whose result is read much
    # later; the atomic optimizer would broadcast the result right away and
    # make the wave wait for every load issued before the atomic
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


# Kernel instances on the measured hot path that must keep everything in
# registers (a spill to scratch memory inside their loops costs bandwidth):
# the decode-sweep GEMVs and the dequant.  The build fails if one spills.
NO_SPILL = (
    "gemv_wave_kernel<1, 2, 1, 4, true, 0, true>",
    "gemv_wave_kernel<1, 2, 1, 4, false, 0, true>",
    "gemv_xlds_kernel<1, 2, 3, 3, 0>",
    "gemv_xlds_kernel<1, 2, 3, 3, 1>",
    "gemv_xlds_kernel<1, 2, 3, 3, 2>",
    "dequant_vec_kernel<0, 4, 0>",
    "dequant_vec_kernel<1, 4, 0>",
    "gemv_stream_kernel<4, 1, 4, 4, 0, true, 2, true>",
    "gemv_stream_kernel<8, 2, 4, 2, 0, true, 2, true>",
)
RESOURCES = os.path.join(PKG, "kernel_resources.txt")
REMARKS = "-Rpass-analysis=kernel-resource-usage"


def parse_resources(text: str) -> dict:
    """Kernel name -> {VGPRs, AGPRs, ScratchSize, Occupancy, LDS} from the
    compiler's kernel-resource-usage remarks (names demangled by c++filt)."""
    import re
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out.setdefault(cur, {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur:
            out[cur][keys[m.group(1)]] = int(m.group(2))
    names = list(out)
    if names and shutil.which("c++filt"):
        res = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        demangled = res.stdout.splitlines()
        if len(demangled) == len(names):
            out = {d: out[n] for n, d in zip(names, demangled)}
    return out


def write_resources(res: dict) -> list:
    """Writes the per-kernel table to kernel_resources.txt; returns the hot
    instances (NO_SPILL) that use scratch."""
    rows = sorted(res.items())
    with open(RESOURCES, "w", encoding="utf-8") as f:
        f.write("# per-kernel resources from the compiler (hipcc -Rpass-analysis="
                "kernel-resource-usage)\n# vgpr agpr scratch[B/lane] occupancy[waves/SIMD] "
                "lds[B/block]  kernel\n")
        for name, r in rows:
            f.write(f"{r.get('vgpr', -1):4d} {r.get('agpr', -1):4d} {r.get('scratch', -1):5d} "
                    f"{r.get('occupancy', -1):2d} {r.get('lds', -1):7d}  {name}\n")
    bad = []
    for hot in NO_SPILL:
        for name, r in rows:
            if hot in name and r.get("scratch", 0) > 0:
                bad.append(f"{name}: {r['scratch']} bytes of scratch per lane")
    return bad


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnf4)")


def build(verbose: bool = False, cached: bool = False) -> str:
    """Compile each source to an object in parallel (one hipcc per file), then
    link the shared library; the result replaces LIB atomically.  cached:
    reuse the object of a source whose content, headers and flags are
    unchanged since it was last compiled (off by default: a build compiles
    every source)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    import hashlib
    tmp = tempfile.mkdtemp(prefix="nf4_build_")
    # objects (and their compiler remarks) are kept per content hash of the
    # source, every header and the flags, so an unchanged source is not
    # recompiled
    cache = os.path.join(tempfile.gettempdir(), "nf4_build_cache")
    os.makedirs(cache, exist_ok=True)
    headers = b""
    for d in (os.path.join(PKG, "csrc"), INCLUDE):
        for fn in sorted(os.listdir(d)):
            if fn.endswith(".h"):
                with open(os.path.join(d, fn), "rb") as f:
                    headers += fn.encode() + f.read()
    try:
        objs, cmds, keys = [], [], []
        for src in SRCS:
            with open(src, "rb") as f:
                h = hashlib.sha256(f.read() + headers + " ".join(HIPCC_FLAGS).encode() +
                                   hipcc().encode()).hexdigest()[:24]
            keys.append(os.path.join(cache, f"{os.path.basename(src)}.{h}"))
            objs.append(os.path.join(tmp, os.path.basename(src) + ".o"))
            cmds.append([hipcc(), *HIPCC_FLAGS, REMARKS, "-I", INCLUDE, "-c", "-o", objs[-1], src])

        def compile_one(i):
            key = keys[i]
            if cached and os.path.exists(key + ".o") and os.path.exists(key + ".remarks"):
                shutil.copyfile(key + ".o", objs[i])
                with open(key + ".remarks", encoding="utf-8") as f:
                    return subprocess.CompletedProcess(cmds[i], 0, "", f.read())
            if verbose:
                print(" ".join(cmds[i]), flush=True)
            res = subprocess.run(cmds[i], capture_output=True, text=True)
            if res.returncode == 0:
                shutil.copyfile(objs[i], key + ".o.tmp")
                os.replace(key + ".o.tmp", key + ".o")
                with open(key + ".remarks", "w", encoding="utf-8") as f:
                    f.write(res.stderr)
            return res

        with ThreadPoolExecutor(len(cmds)) as pool:
            results = list(pool.map(compile_one, range(len(cmds))))
        for res in results:
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed to build libnf4.so")
        resources = {}
        for res in results:
            resources.update(parse_resources(res.stderr))
        spills = write_resources(resources)
        if verbose:
            spilling = sum(1 for r in resources.values() if r.get("scratch", 0) > 0)
            print(f"{len(resources)} kernels, {spilling} with scratch; table in {RESOURCES}",
                  flush=True)
        if spills:
            raise RuntimeError("hot-path kernel instances spill to scratch:\n  " +
                               "\n  ".join(spills))
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed to link libnf4.so")
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, cached="--cached" in sys.argv))
