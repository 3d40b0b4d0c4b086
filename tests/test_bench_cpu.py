"""Host-side logic of bench.py, on the CPU: the refusal of more than one GPU,
the algorithmic byte count of each kernel on a routing worked by hand, and
the rule that counter-based traffic is reported only for the kernel sources
it was measured on."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_by_hand():
    # 3 tokens x top-2 over 2 experts, hidden 128, BLOCK_M 4: token 0 -> expert 0
    # (slot 1 masked), token 1 -> experts 1 and 0, token 2 fully masked.
    cfg = CONFIGS["tiny"].replace(tokens=3, top_k=2, hidden=128, num_experts=2,
                                  experts_global=2, block_m=4)
    idx = np.array([[0, -1], [1, 0], [-1, -1]], dtype=np.int32)
    counts = np.array([2, 1], dtype=np.int32)
    # N_a = 3 real rows, T_act = 2 active tokens, capacity 6 + 2 * 3 = 12 rows
    bf = bench.algorithmic_bytes(cfg, idx, counts, fp8=False)
    assert (bf["n_a"], bf["t_act"], bf["pool_rows"]) == (3, 2, 8)
    assert bf["layout"] == 16 * 6 + 4 * 12                       # 144
    assert bf["dispatch"] == 4 * 6 + 2 * 128 * 2 + 2 * 128 * 3   # 1304
    assert bf["combine"] == 8 * 6 + 2 * 128 * 3 + 2 * 128 * 3    # 1584
    f8 = bench.algorithmic_bytes(cfg, idx, counts, fp8=True)
    # FP8 rows are one byte per channel plus one scale byte per 128 channels
    assert f8["dispatch"] == 4 * 6 + 2 * 128 * 2 + 128 * 3 + 3   # 923
    assert f8["combine"] == bf["combine"] and f8["layout"] == bf["layout"]


def test_traffic_needs_the_measured_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.kernel_source_sha()
    body = "kernel: k\nworkload: w\ntraffic_bytes_per_launch: 123456\nsource_sha: {}\n"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))           # summaries read from here
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)  # the sources stay this tree's
    assert bench.read_traffic("dispatch", "prefill", 1.0) is None          # no summary
    (prof / "traffic_dispatch_prefill.txt").write_text(body.format(sha))
    assert bench.read_traffic("dispatch", "prefill", 1.0) == 123456.0
    (prof / "traffic_dispatch_prefill.txt").write_text(body.format("0" * 16))
    assert bench.read_traffic("dispatch", "prefill", 1.0) is None          # other sources


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The hash that ties counter summaries to the kernels is taken over the
    sources with comments and blank space removed: a comment edit keeps it,
    a code edit changes it."""
    import shutil
    src = os.path.join(ROOT, "combine_ep_layout_amd", "csrc")
    dst = tmp_path / "combine_ep_layout_amd" / "csrc"
    shutil.copytree(src, dst)
    here = bench.kernel_source_sha()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_sha() == here
    k = dst / "ep_kernels.hip"
    text = k.read_text()
    k.write_text(text.replace("namespace epk {", "// a new comment\nnamespace epk {  /* and another */", 1))
    assert bench.kernel_source_sha() == here
    k.write_text(text.replace("constexpr int kDispatchChunks = 2;", "constexpr int kDispatchChunks = 3;", 1))
    assert bench.kernel_source_sha() != here
