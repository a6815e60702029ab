"""Build the oracle's one C routine (canonical float32 router logits) with gcc.

Test infrastructure: the shared object it writes is loaded only by the oracle.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "router_logits.c")
LIB = os.path.join(HERE, "_liboracle.so")

# -ffp-contract=off: the only fused multiply-adds are the explicit fmaf() calls.
# -mfma lets gcc emit the hardware instruction for fmaf (correctly rounded either way).
CFLAGS = ["-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
