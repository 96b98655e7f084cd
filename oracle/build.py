"""Build the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is compiled here so that the test suite, the
smoke check and the benchmark's CPU-baseline leg can load it.  Strict IEEE
fp32 arithmetic: no fused multiply-add contraction, no fast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nf4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fopenmp", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
