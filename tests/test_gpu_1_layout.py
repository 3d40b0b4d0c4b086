"""GPU parity of the layout kernels against the oracle: every metadata array
bit-exact (StreamEP README, "Streaming dispatch in one paragraph")."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate
from gpu_helpers import (say, inputs, oracle_layout, new_handle, device_routing, compare_layout)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "decode", "share", "prefill", "stream"])
def test_layout_full_size(name):
    import combine_ep_layout_amd as ep
    say(f"[layout] {name} full size")
    cfg, d = inputs(name)
    L = oracle_layout(name)
    h = new_handle(cfg)
    idx, w = device_routing(d)
    h.layout(idx, w)
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    compare_layout(h, L)
    assert torch.equal(h.array("topk_weights").cpu(), torch.from_numpy(d["topk_weights"]).view(-1))
    counts, nt = h.counts_to_host()
    assert np.array_equal(counts, L["expert_counts"]) and nt == L["num_tiles"]
    h.close()


@pytest.mark.parametrize("name,tokens", [("prefill", 5000), ("stream", 3001), ("share", 2049),
                                         ("decode", 2047)])
def test_layout_ragged_sizes(name, tokens):
    # multi-workgroup path with a partial last workgroup, and the single-workgroup
    # path just below its slot limit
    say(f"[layout] {name} tokens={tokens}")
    cfg = CONFIGS[name].replace(tokens=tokens, hidden=128)
    d = generate(cfg, 3)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    compare_layout(h, L)
    h.close()


def test_layout_many_experts_single_workgroup_count():
    # more experts than the single-workgroup path takes, with few slots
    say("[layout] E=1000 few slots")
    cfg = CONFIGS["tiny"].replace(tokens=40, hidden=128, num_experts=1000, experts_global=1000,
                                  top_k=4, block_m=3)
    d = generate(cfg, 1)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    compare_layout(h, L)
    h.close()


def test_layout_reuse_handle_new_routing():
    # a second layout on the same handle fully replaces the first
    say("[layout] reuse handle")
    cfg = CONFIGS["stream"].replace(tokens=6000, hidden=128)
    h = new_handle(cfg)
    for seed in (0, 1, 2):
        d = generate(cfg, seed)
        n = 6000 - 1000 * seed
        d = {k: v[:n] for k, v in d.items()}
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m,
                          cap=oracle.capacity_rows(6000, cfg.top_k, cfg.num_experts, cfg.block_m))
        e = h.layout(*device_routing(d))
        assert e == seed + 1
        compare_layout(h, L)
    h.close()
