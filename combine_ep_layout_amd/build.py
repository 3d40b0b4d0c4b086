"""Build libep_layout.so (gfx950) in-tree with hipcc.

    python combine_ep_layout_amd/build.py [-v] [-DNAME=VALUE ...] [-o OUT]

(run as a script: importing the package would load the library it builds)

Extra -D options override the kernels' compile-time tuning macros.
"""
from __future__ import annotations

import os
import subprocess
import sys
from typing import Iterable, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libep_layout.so")
SOURCES = [os.path.join(CSRC, "ep_kernels.hip"), os.path.join(CSRC, "ep_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms stay off; scalar fp32 code is used throughout
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 denormals are kept (the dequant path produces them)
    "-fno-gpu-flush-denormals-to-zero",
    # the combine's fused multiply-adds are explicit; nothing else is contracted
    "-ffp-contract=off",
    # float32 division is IEEE (the FP8 float32-scale flavour divides)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
    "-Wno-unused-variable",
    "-Wno-unused-parameter",
]


def build(verbose: bool = False, defines: Iterable[str] = (), out: Optional[str] = None) -> str:
    out = out or LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *defines, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out = None
    if "-o" in args:
        i = args.index("-o")
        out = args[i + 1]
        del args[i:i + 2]
    defs = [a for a in args if a.startswith("-D")]
    print(build(verbose="-v" in args, defines=defs, out=out))
