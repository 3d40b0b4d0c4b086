"""Parity at the limits the C ABI accepts: hidden 65536, 1024 experts (fused
and multi-workgroup layout), BLOCK_M 4096, and the largest token count
(2^19 tokens x top-32, 16.8 M slots) through layout, dispatch and combine.
The small cases compare every output with the oracle as the other parity
tests do.  The largest one compares every layout array, every pool row on
the device against the row of x it came from, and every token of combine."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (say, dev, new_handle, device_routing, compare_layout, full_path_check,
                         bits_of, ulp_diff)
from synth import Config, generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fp8", [False, True])
def test_hidden_max(fp8):
    """Rows of 65536 channels: 19 bf16 dispatch segments (the last one
    partial), 64 combine segments, 512 FP8 groups per row."""
    say(f"[limits] hidden 65536 fp8={fp8}")
    cfg = Config("hidden_max", 6, 65536, 3, 5, 5, 4)
    full_path_check(cfg, generate(cfg, 3), fp8=fp8)


@pytest.mark.parametrize("tokens,block_m", [(200, 1), (200, 128), (700, 1), (700, 128)])
def test_experts_max(tokens, block_m):
    """1024 experts: 1600 slots take the one-workgroup layout, 5600 slots the
    multi-workgroup one (three workgroups, per-wave LDS counters for every
    expert)."""
    say(f"[limits] 1024 experts, {tokens} tokens, BLOCK_M {block_m}")
    cfg = Config("experts_max", tokens, 128, 8, 1024, 1024, block_m)
    full_path_check(cfg, generate(cfg, 4))


@pytest.mark.parametrize("fp8", [False, True])
def test_block_m_max(fp8):
    """BLOCK_M 4096 with four experts: one tile each, mostly padding."""
    say(f"[limits] BLOCK_M 4096 fp8={fp8}")
    cfg = Config("block_m_max", 1000, 256, 3, 4, 4, 4096)
    full_path_check(cfg, generate(cfg, 5), fp8=fp8)


def test_max_tokens_top32():
    """2^19 tokens x top-32 over 1024 experts (masked slots and repeated
    experts included): the largest grids and row indices the ABI allows."""
    import combine_ep_layout_amd as ep
    T, K, E, BM, H = 1 << 19, 32, 1024, 128, 128
    say(f"[limits] {T} tokens x top-{K}, {E} experts")
    rng = np.random.default_rng(6)
    idx = rng.integers(-1, E, size=(T, K), dtype=np.int32)
    w = rng.random((T, K), dtype=np.float32)
    L = oracle.layout(idx, E, BM)
    h = ep.EpHandle(T, K, E, BM)
    epoch = h.layout(torch.from_numpy(idx).to(dev()), torch.from_numpy(w).to(dev()))
    compare_layout(h, L)
    assert np.array_equal(h.array("topk_weights").cpu().numpy().view(np.float32), w.ravel())
    say("  layout matches")
    # dispatch: every real row equals the row of x it came from, padding untouched
    cap = h.capacity_rows
    g = torch.Generator(device=dev())
    g.manual_seed(7)
    x = torch.randn(T, H, generator=g, device=dev()).to(torch.bfloat16)
    pool = torch.full((cap, H), -0x4111, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    h.dispatch(x, pool, None)
    recv = torch.from_numpy(L["pool_recv_token"]).to(dev())
    real = recv >= 0
    assert torch.equal(pool.view(torch.int16)[real], x.view(torch.int16)[recv[real].long()])
    assert bool((pool.view(torch.int16)[~real] == -0x4111).all())
    del pool
    say("  dispatch matches")
    # combine on seeded expert rows, NaN in every row no slot owns: every
    # token against the oracle (top-32 walks the slots in four groups of 8)
    from oracle import par as oracle_par
    eo = torch.randn(cap, H, generator=g, device=dev()).to(torch.bfloat16)
    eo[~real] = float("nan")
    y = h.combine(epoch, eo)
    eo_h = bits_of(eo)
    del eo
    y_or = oracle_par.combine(eo_h, L["slot_to_pool_row"], w)
    del eo_h
    diff = ulp_diff(bits_of(y), y_or)
    say(f"  combine: non-identical elements {(diff > 0).sum()} of {diff.size}")
    assert diff.max() <= 1
    assert h.sync_status() == ep.EP_OK
    h.close()


@pytest.mark.parametrize("kind,mn", [("ue8m0", False), ("f32", True)])
def test_cast_back_grid_stride(kind, mn):
    """A cast back of more work items than the grid holds (4.3 M rows of one
    128-channel group: 4.3 M one-wave items against a grid capped at 2^20
    four-wave workgroups), so some waves take a second item and reuse their
    LDS staging.  Rows at the start, around the wrap point (item 4 * 2^20)
    and at the end, and a random sample, against the oracle bit for bit."""
    import combine_ep_layout_amd as ep
    rows, H = 4_300_000, 128
    say(f"[limits] cast back grid stride kind={kind} mn={mn} rows={rows}")
    g = torch.Generator(device=dev())
    g.manual_seed(13)
    q = torch.randint(0, 256, (rows, H), generator=g, device=dev(), dtype=torch.int32).to(torch.uint8)
    if kind == "ue8m0":
        rm = torch.randint(100, 160, (rows, 1), generator=g, device=dev(), dtype=torch.int32).to(torch.uint8)
    else:
        rm = torch.rand((rows, 1), generator=g, device=dev()) + 0.01
    # MN-major float scales: [groups, ld] with ld = rows
    s_dev = rm.t().contiguous() if mn else rm
    out = ep.cast_back(q, s_dev, kind, mn, rows=rows)
    wrap = 4 * (1 << 20)
    rng = np.random.default_rng(3)
    pick = np.unique(np.concatenate([np.arange(0, 2000), np.arange(wrap - 1000, wrap + 1000),
                                     np.arange(rows - 2000, rows), rng.integers(0, rows, 5000)]))
    idx = torch.from_numpy(pick).to(dev())
    q_h = q[idx].cpu().numpy()
    s_h = rm[idx].cpu().numpy()
    want = oracle.cast_back(q_h, s_h, kind, False)
    assert np.array_equal(bits_of(out[idx]), want)
