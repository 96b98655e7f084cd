"""Build libnf4.so (the gfx950 HIP library) in-tree with hipcc.

Flags:
  --offload-arch=gfx950     CDNA4 only; no other targets, no host fallback.
  -ffp-contract=off         the dequant formula rounds each product and sum to
                            fp32 on its own; GEMV code uses explicit fmaf.
  -target-feature -packed-fp32-ops
                            no packed fp32 VALU instructions.
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


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnf4)")


def build(verbose: bool = False) -> str:
    """Compile each source to an object in parallel (one hipcc per file), then
    link the shared library; the result replaces LIB atomically."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    tmp = tempfile.mkdtemp(prefix="nf4_build_")
    try:
        objs = [os.path.join(tmp, os.path.basename(src) + ".o") for src in SRCS]
        cmds = [[hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-c", "-o", obj, src]
                for src, obj in zip(SRCS, objs)]
        if verbose:
            for cmd in cmds:
                print(" ".join(cmd), flush=True)
        with ThreadPoolExecutor(len(cmds)) as pool:
            results = list(pool.map(lambda c: subprocess.run(c, capture_output=True, text=True),
                                    cmds))
        for res in results:
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed to build libnf4.so")
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
    print(build(verbose="-v" in sys.argv))
