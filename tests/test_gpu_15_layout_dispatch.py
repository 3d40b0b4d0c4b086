"""ep_layout_dispatch (the layout and the dispatch in one call, one kernel
launch for at most 2048 slots) against the oracle and against the two calls
made one after the other on a second handle: every layout array, every pool
row and scale, the untouched padding, the epoch and sequence numbers, and a
combine afterwards."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate, expert_rows
from gpu_helpers import (say, new_handle, device_routing, to_dev_bf16, bits_of, compare_layout, dev,
                         ulp_diff, POISON_BF16, POISON_U8, LAYOUT_ARRAYS)

pytestmark = pytest.mark.gpu


def _pool(h, H, fp8, kind="ue8m0", mn=False):
    """A pool (and scales) of the handle's capacity, every byte poisoned."""
    if not fp8:
        return (torch.full((h.capacity_rows, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev())
                .view(torch.bfloat16), None)
    pool, scales = h.new_pool(H, fp8=True, scale_kind=kind, mn_major=mn)
    pool.fill_(POISON_U8)
    scales.view(torch.uint8).fill_(POISON_U8)
    return pool, scales


def _check(cfg, d, fp8, kind="ue8m0", mn=False, seed=0):
    import combine_ep_layout_amd as ep
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    idx, w = device_routing(d)
    x = to_dev_bf16(d["x"])
    # the fused call
    h1 = new_handle(cfg)
    pool1, sc1 = _pool(h1, H, fp8, kind, mn)
    epoch1, seq1 = h1.layout_dispatch(idx, w, x, pool1, sc1, fp8=fp8, scale_kind=kind, mn_major=mn)
    # the two calls
    h2 = new_handle(cfg)
    pool2, sc2 = _pool(h2, H, fp8, kind, mn)
    epoch2 = h2.layout(idx, w)
    seq2 = h2.dispatch(x, pool2, sc2, fp8=fp8, scale_kind=kind, mn_major=mn)
    torch.cuda.synchronize()
    assert (epoch1, seq1) == (epoch2, seq2)
    compare_layout(h1, L)
    for name in LAYOUT_ARRAYS + ["num_tiles", "topk_weights", "tile_ready", "pool_arrival_count"]:
        assert torch.equal(h1.array(name), h2.array(name)), name
    real = torch.from_numpy(np.flatnonzero(L["pool_recv_token"] >= 0)).to(dev())
    pad = torch.from_numpy(np.flatnonzero(L["pool_recv_token"] < 0)).to(dev())
    p1 = pool1.view(torch.uint8) if fp8 else pool1.view(torch.int16)
    p2 = pool2.view(torch.uint8) if fp8 else pool2.view(torch.int16)
    assert torch.equal(p1, p2)
    if fp8:
        assert torch.equal(sc1.view(torch.uint8), sc2.view(torch.uint8))
        if kind == "ue8m0" and not mn:
            op, osc = oracle.dispatch_fp8(d["x"], L["pool_recv_token"],
                                          pool_init=np.full(tuple(pool1.shape), POISON_U8, np.uint8),
                                          scales_init=np.full(tuple(sc1.shape), POISON_U8, np.uint8))
            assert np.array_equal(pool1.cpu().numpy(), op)
            assert np.array_equal(sc1.cpu().numpy(), osc)
    else:
        src = torch.from_numpy(L["pool_recv_token"][L["pool_recv_token"] >= 0].astype(np.int64)).to(dev())
        assert torch.equal(p1[real], x.view(torch.int16)[src])
        assert bool((p1[pad] == POISON_BF16 - 0x10000).all())
    # a combine on the fused handle's layout
    cap = h1.capacity_rows
    o_slot = expert_rows(T, K, H, seed=seed + 5)
    eo = np.full((cap, H), 0x7FC0, np.uint16)
    s2r = L["slot_to_pool_row"].reshape(T, K)
    valid = s2r >= 0
    eo[s2r[valid]] = o_slot[valid]
    y = h1.combine(epoch1, to_dev_bf16(eo))
    y_or = oracle.combine(eo, L["slot_to_pool_row"], d["topk_weights"])
    assert ulp_diff(bits_of(y), y_or).max(initial=0) <= 1
    want = ep.EP_ERR_BAD_ROUTING if L["error"] else ep.EP_OK
    assert h1.sync_status() == want and h2.sync_status() == want
    h1.close()
    h2.close()


@pytest.mark.parametrize("name,tokens,hidden,fp8", [
    ("decode", -1, -1, True),        # 256 tokens x top-8: 2048 slots, one launch
    ("decode", 100, 1024, True),
    ("decode", 256, 1024, False),
    ("tiny", -1, -1, False),
    ("prefill", 200, 1152, False),   # Zipf routing, 256 experts
    ("decode", 300, 512, True),      # 2400 slots: the two calls
])
def test_layout_dispatch_equals_two_calls(name, tokens, hidden, fp8):
    cfg = CONFIGS[name]
    if tokens >= 0:
        cfg = cfg.replace(tokens=tokens)
    if hidden >= 0:
        cfg = cfg.replace(hidden=hidden)
    say(f"[layout+dispatch] {name} tokens={cfg.tokens} hidden={cfg.hidden} fp8={fp8}")
    _check(cfg, generate(cfg, 11), fp8)


@pytest.mark.parametrize("kind,mn", [("f32", False), ("pow2_f32", False), ("ue8m0", True), ("f32", True)])
def test_layout_dispatch_scale_flavours(kind, mn):
    cfg = CONFIGS["decode"].replace(tokens=192, hidden=1024)
    say(f"[layout+dispatch] decode 192 tokens, scales {kind} mn_major={mn}")
    _check(cfg, generate(cfg, 12), True, kind, mn)


@pytest.mark.parametrize("top_k,tokens", [(1, 2048), (2, 1000), (4, 512), (16, 128), (32, 64), (32, 70)])
def test_layout_dispatch_top_k(top_k, tokens):
    """Every slot group size the kernels take, up to the 2048-slot limit of
    the one-launch path (32 x 70 = 2240 slots take the two calls)."""
    cfg = CONFIGS["decode"].replace(tokens=tokens, hidden=512, top_k=top_k, num_experts=48,
                                    experts_global=48)
    for fp8 in (False, True):
        say(f"[layout+dispatch] top_k={top_k} tokens={tokens} fp8={fp8}")
        _check(cfg, generate(cfg, 13 + top_k), fp8)


def test_layout_dispatch_masked_and_bad_ids():
    """Masked slots, a token with none left, and ids outside [-1, E), which
    the layout flags in the error word."""
    cfg = CONFIGS["decode"].replace(tokens=64, hidden=512)
    d = dict(generate(cfg, 21))
    idx = d["topk_idx"].copy()
    idx[3, :] = -1
    idx[5, 2] = cfg.num_experts + 3
    idx[9, ::2] = -1
    d["topk_idx"] = idx
    say("[layout+dispatch] masked slots and a bad id")
    _check(cfg, d, True)


def test_layout_dispatch_then_more_calls():
    """The handle after a fused call behaves as after the two calls: a
    streaming dispatch on the same layout (round 1), a new fused call (new
    epoch), and an empty batch."""
    import combine_ep_layout_amd as ep
    cfg = CONFIGS["decode"].replace(tokens=128, hidden=512)
    d = generate(cfg, 31)
    idx, w = device_routing(d)
    x = to_dev_bf16(d["x"])
    h = new_handle(cfg)
    pool, sc = _pool(h, cfg.hidden, True)
    e1, s1 = h.layout_dispatch(idx, w, x, pool, sc, fp8=True)
    s2 = h.dispatch(x, pool, sc, fp8=True, tile_ready=True)
    torch.cuda.synchronize()
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    nt = L["num_tiles"]
    assert s2 == s1 + 1
    assert (h.array("tile_ready").cpu().numpy().view(np.uint32)[:nt] == s2).all()
    assert np.array_equal(h.array("pool_arrival_count").cpu().numpy()[:nt].view(np.uint32),
                          L["pool_arrival_target"][:nt].astype(np.uint32))
    e3, s3 = h.layout_dispatch(idx[:0], w[:0], x[:0], pool, sc, fp8=True)
    assert (e3, s3) == (e1 + 1, s2 + 1)
    assert h.num_tokens == 0
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_layout_dispatch_rejections():
    import ctypes
    import combine_ep_layout_amd as ep
    lib = ep.library()
    cfg = CONFIGS["decode"].replace(tokens=64, hidden=512)
    d = generate(cfg, 41)
    idx, w = device_routing(d)
    x = to_dev_bf16(d["x"])
    h = new_handle(cfg)
    pool, sc = _pool(h, cfg.hidden, True)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    e, s = ctypes.c_uint32(), ctypes.c_uint32()
    call = lambda *a: lib.ep_layout_dispatch(h.raw, *a, None, ctypes.byref(e), ctypes.byref(s))
    assert call(P(idx), P(w), 64, P(x), 512, P(pool), P(sc), ep.EP_DISPATCH_FP8 | ep.EP_DISPATCH_BORROW) \
        == ep.EP_ERR_UNSUPPORTED
    assert call(P(idx), P(w), 65, P(x), 512, P(pool), P(sc), ep.EP_DISPATCH_FP8) == ep.EP_ERR_INVALID_ARGUMENT
    assert call(P(idx), P(w), 64, P(x), 500, P(pool), P(sc), ep.EP_DISPATCH_FP8) == ep.EP_ERR_INVALID_ARGUMENT
    assert call(P(idx), P(w), 64, P(x), 512, P(pool), None, ep.EP_DISPATCH_FP8) == ep.EP_ERR_INVALID_ARGUMENT
    assert call(P(idx), P(w), 64, P(x), 512, P(pool), P(sc), 0) == ep.EP_ERR_INVALID_ARGUMENT
    assert call(None, P(w), 64, P(x), 512, P(pool), P(sc), ep.EP_DISPATCH_FP8) == ep.EP_ERR_INVALID_ARGUMENT
    # nothing was enqueued and the handle has no layout yet
    assert h.num_tokens < 0
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_layout_dispatch_in_graph():
    """ep_layout_dispatch + ep_combine captured in a HIP graph and replayed on
    new inputs written into the captured buffers: every replay's layout,
    pool, scales and y equal an eager run's (two fused calls per replay)."""
    import combine_ep_layout_amd as ep
    say("[layout+dispatch] captured in a graph, 3 replays")
    cfg = CONFIGS["decode"].replace(tokens=200, hidden=1024)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    cap = h.capacity_rows
    idx = torch.empty(T, K, dtype=torch.int32, device=dev())
    w = torch.empty(T, K, dtype=torch.float32, device=dev())
    x = torch.empty(T, H, dtype=torch.bfloat16, device=dev())
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    pool, sc = _pool(h, H, True)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev())

    def load(seed):
        d = generate(cfg, seed)
        idx.copy_(torch.from_numpy(d["topk_idx"]))
        w.copy_(torch.from_numpy(d["topk_weights"]))
        x.copy_(to_dev_bf16(d["x"]))
        eo.copy_(torch.randn(cap, H, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16))
        return d

    def step():
        e, _ = h.layout_dispatch(idx, w, x, pool, sc, fp8=True)
        h.combine(e, eo, y)

    load(0)
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    h.set_density_hint(ep.EP_DENSITY_DENSE)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        d = load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (h.array("slot_to_pool_row").clone(), pool.clone(), sc.clone(), y.clone())
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], h.array("slot_to_pool_row"))
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
        assert np.array_equal(got[0].cpu().numpy(), L["slot_to_pool_row"])
        assert torch.equal(got[1], pool) and torch.equal(got[2], sc)
        assert torch.equal(got[3].view(torch.int16), y.view(torch.int16))
        say(f"  replay with seed {seed} matches the eager step")
    assert h.sync_status() == ep.EP_OK
    del g
    h.close()
