"""The C ABI driven by a plain C program (tests/c_abi/ep_c_demo.c, compiled
by build() with gcc against libep_layout.so): handle, layout, dispatch and
combine on hipMalloc'd buffers, with no Python or torch in that process.  The
program checks its results against exact properties (expert counts against a
host histogram, every pool row against its row of x, identity experts with
weights 1/2 giving x, x/2 or +0 back) and prints one "ok" line."""
import os
import subprocess

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "ep_c_demo")


def test_plain_c_program_end_to_end():
    assert os.path.exists(EXE), "tests/c_abi/ep_c_demo is built by __graft_entry__.build()"
    say("[c abi] running tests/c_abi/ep_c_demo as a child process")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    if r.stderr.strip():
        say(r.stderr.strip()[-2000:])
    assert r.returncode == 0
    assert r.stdout.startswith("c abi demo ok")
