"""Build the CPU oracle shared library (gcc, no fast-math, no contraction).

Test infrastructure: the HIP library neither builds nor loads this.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "libep_oracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile `src` (the oracle's C source, or a copy of it) into `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
