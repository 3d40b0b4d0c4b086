"""Build libep_layout.so (gfx950) in-tree with hipcc, and beside it
libep_ceiling.so, the bandwidth probes the benchmark's ceiling leg loads.

    python combine_ep_layout_amd/build.py [-v] [-o OUT]

(run as a script: importing the package would load the library it builds)
"""
from __future__ import annotations

import os
import subprocess
import sys
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libep_layout.so")
SOURCES = [os.path.join(CSRC, "ep_kernels.hip"), os.path.join(CSRC, "ep_api.hip"),
           os.path.join(CSRC, "ep_noalloc.hip")]
CEILING_LIB = os.path.join(PKG, "libep_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "ep_ceiling.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 VALU forms (v_pk_*_f32) in the device code: without this
    # the gfx950 build has ~3500 of them, with it none.  The host pass does
    # not know the feature and says it ignores it; that warning is harmless.
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


def _hipcc(out: str, sources: list, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, out: Optional[str] = None) -> str:
    """Builds the library (to `out` if given) and the probe library; returns
    the library's path."""
    _hipcc(CEILING_LIB, CEILING_SOURCES, verbose)
    return _hipcc(out or LIB, SOURCES, verbose)


if __name__ == "__main__":
    args = sys.argv[1:]
    out = None
    if "-o" in args:
        i = args.index("-o")
        out = args[i + 1]
        del args[i:i + 2]
    print(build(verbose="-v" in args, out=out))
