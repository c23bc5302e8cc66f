"""Build the CPU oracle's shared library (plain gcc, scalar, no fast-math).

Test infrastructure only: the GPU library never links or loads it.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add anywhere, so every fp32 step is
# the single IEEE operation written in the source. x86-64 evaluates float in
# SSE registers (no excess precision).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
