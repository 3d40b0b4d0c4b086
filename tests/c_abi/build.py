"""Build the plain-C user of the C ABI (ep_c_demo) against the in-tree
libep_layout.so with gcc.

    python tests/c_abi/build.py [-v]

The library must be built first (combine_ep_layout_amd/build.py).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "ep_c_demo.c")
EXE = os.path.join(HERE, "ep_c_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "combine_ep_layout_amd"), "-lep_layout",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           # found next to the package wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../combine_ep_layout_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
