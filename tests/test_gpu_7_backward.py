"""GPU parity of the backward calls against the oracle (StreamEP README, "What's
in the box": dispatch_grads / combine_grads).  Gradient rows and grad_x are
bit-exact; grad_w is the exact dot product rounded once to float, computed in
double in a different summation order than the oracle's, so it must agree
within one float ulp plus 2*H*2^-53*sum|g*o| (the double rounding of both
orders)."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Config, generate, expert_rows, bf16_to_f32
from gpu_helpers import (say, inputs, new_handle, device_routing, to_dev_bf16, bits_of, dev,
                         POISON_BF16)

pytestmark = pytest.mark.gpu


def _rows_and_grads(cfg, L, seed=3):
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    o_slot = expert_rows(T, K, H, seed=seed)
    eo = np.full((L["capacity_rows"], H), 0x7FC0, np.uint16)       # padding is NaN
    s2r = L["slot_to_pool_row"].reshape(T, K)
    valid = s2r >= 0
    eo[s2r[valid]] = o_slot[valid]
    gy = expert_rows(T, 1, H, seed=seed + 1)[:, 0, :]
    return eo, gy, s2r, valid


def _check_grad_w(got, want, gy, eo, s2r, valid, chunk=512):
    H = gy.shape[1]
    assert (got[~valid] == 0).all()
    differ = 0
    for t0 in range(0, gy.shape[0], chunk):              # bounded host memory at full size
        t1 = min(gy.shape[0], t0 + chunk)
        ts, ks = np.nonzero(valid[t0:t1])
        ts = ts + t0
        g64 = bf16_to_f32(gy[ts]).astype(np.float64)
        o64 = bf16_to_f32(eo[s2r[ts, ks]]).astype(np.float64)
        absum = np.abs(g64 * o64).sum(1)
        w = want[ts, ks].astype(np.float64)
        bound = np.spacing(np.abs(want[ts, ks])).astype(np.float64) + 2 * H * 2.0 ** -53 * absum
        diff = np.abs(got[ts, ks].astype(np.float64) - w)
        assert np.all(diff <= bound), t0
        differ += int((diff > 0).sum())
    return differ


@pytest.mark.parametrize("name,tokens", [("tiny", -1), ("decode", -1), ("share", -1),
                                         ("prefill", 1000), ("stream", 2000)])
def test_combine_backward_parity(name, tokens):
    say(f"[backward] combine {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    eo, gy, s2r, valid = _rows_and_grads(cfg, L)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    cap, H = h.capacity_rows, cfg.hidden
    geo = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    _, gw = h.combine_backward(epoch, to_dev_bf16(gy), to_dev_bf16(eo), geo)
    geo_or, gw_or = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], d["topk_weights"],
                                            grad_eo_init=np.full((cap, H), POISON_BF16, np.uint16))
    assert np.array_equal(bits_of(geo), geo_or)                 # rows bit-exact, others untouched
    n = _check_grad_w(gw.cpu().numpy(), gw_or, gy, eo, s2r, valid)
    say(f"  grad_w not bit-identical: {n} of {int(valid.sum())}")
    h.close()


@pytest.mark.parametrize("name,tokens", [("tiny", -1), ("decode", -1), ("share", -1),
                                         ("prefill", 1000), ("stream", 2000)])
def test_dispatch_backward_parity(name, tokens):
    say(f"[backward] dispatch {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    gp, _, _, _ = _rows_and_grads(cfg, L, seed=7)                 # NaN padding is never read
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    gx = h.dispatch_backward(epoch, to_dev_bf16(gp))
    want = oracle.dispatch_backward(gp, L["slot_to_pool_row"], cfg.tokens, cfg.top_k)
    assert np.array_equal(bits_of(gx), want)
    h.close()


def test_backward_full_size():
    """The metric's workload at full size: every gradient row, every weight
    gradient and every row of grad_x against the oracle."""
    from oracle import par as oracle_par
    say("[backward] prefill full size, every token")
    cfg, d = inputs("prefill")
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    cap = h.capacity_rows
    g = torch.Generator(device=dev())
    g.manual_seed(77)
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    for r0 in range(0, cap, 16384):
        r1 = min(cap, r0 + 16384)
        eo[r0:r1] = torch.randn(r1 - r0, H, generator=g, device=dev()).to(torch.bfloat16)
    recv = torch.from_numpy(L["pool_recv_token"]).to(dev())
    eo[recv < 0] = float("nan")                   # rows no slot owns are never read
    gy = torch.randn(T, H, generator=g, device=dev()).to(torch.bfloat16)
    geo = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16,
                     device=dev()).view(torch.bfloat16)
    _, gw = h.combine_backward(epoch, gy, eo, geo)
    gx = h.dispatch_backward(epoch, eo)
    eo_h, gy_h = bits_of(eo), bits_of(gy)
    del eo
    geo_or, gw_or = oracle_par.combine_backward(gy_h, eo_h, L["slot_to_pool_row"], d["topk_weights"],
                                                np.full((cap, H), POISON_BF16, np.uint16))
    assert np.array_equal(bits_of(geo), geo_or)           # rows bit-exact, the rest untouched
    del geo, geo_or
    s2r = L["slot_to_pool_row"].reshape(T, K)
    n = _check_grad_w(gw.cpu().numpy(), gw_or, gy_h, eo_h, s2r, s2r >= 0)
    say(f"  grad_w not bit-identical: {n} of {int((s2r >= 0).sum())}")
    gx_or = oracle_par.dispatch_backward(eo_h, L["slot_to_pool_row"], T, K)
    assert np.array_equal(bits_of(gx), gx_or)
    h.close()


@pytest.mark.parametrize("top_k", [16, 32])
def test_backward_top_k_above_8(top_k):
    """top_k 16 and 32: both backward kernels walk a token's slots in groups
    of 8 (combine backward reads grad_y once per group)."""
    say(f"[backward] top_k={top_k}")
    cfg = CONFIGS["stream"].replace(tokens=600, hidden=1024, top_k=top_k, fp8=False,
                                    tile_ready=False)
    d = generate(cfg, 12)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    eo, gy, s2r, valid = _rows_and_grads(cfg, L)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    cap, H = h.capacity_rows, cfg.hidden
    geo = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    _, gw = h.combine_backward(epoch, to_dev_bf16(gy), to_dev_bf16(eo), geo)
    geo_or, gw_or = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], d["topk_weights"],
                                            grad_eo_init=np.full((cap, H), POISON_BF16, np.uint16))
    assert np.array_equal(bits_of(geo), geo_or)
    _check_grad_w(gw.cpu().numpy(), gw_or, gy, eo, s2r, valid)
    gx = h.dispatch_backward(epoch, to_dev_bf16(eo))
    assert np.array_equal(bits_of(gx), oracle.dispatch_backward(eo, L["slot_to_pool_row"],
                                                                 cfg.tokens, top_k))
    h.close()


@pytest.mark.parametrize("name", ["stream", "share"])
def test_combine_backward_every_launch_shape(name):
    """combine_grads runs two workgroups per compute unit for dense routing
    and full occupancy for sparse routing (batches too large to be resident
    at once).  Both shapes forced by the density hint, and the shape the
    layout's report picks, give bit-identical gradient rows and weight
    gradients, which match the oracle (dense: 4096 tokens x top-8 of 128
    experts; sparse: 4096 tokens with 16 of 128 experts kept)."""
    import combine_ep_layout_amd as ep
    cfg = CONFIGS[name].replace(tokens=4096, hidden=1024, fp8=False, tile_ready=False)
    say(f"[backward] every launch shape, {name} routing, {cfg.tokens} tokens")
    d = generate(cfg, 21)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    eo, gy, s2r, valid = _rows_and_grads(cfg, L)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    assert h.layout_density() == (ep.EP_DENSITY_DENSE if name == "stream" else ep.EP_DENSITY_SPARSE)
    cap, H = h.capacity_rows, cfg.hidden
    outs = []
    for hint in (ep.EP_DENSITY_AUTO, ep.EP_DENSITY_DENSE, ep.EP_DENSITY_SPARSE):
        h.set_density_hint(hint)
        geo = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
        _, gw = h.combine_backward(epoch, to_dev_bf16(gy), to_dev_bf16(eo), geo)
        outs.append((bits_of(geo), gw.cpu().numpy()))
    h.set_density_hint(ep.EP_DENSITY_AUTO)
    for geo_b, gw_b in outs[1:]:
        assert np.array_equal(geo_b, outs[0][0])
        assert np.array_equal(gw_b.view(np.uint32), outs[0][1].view(np.uint32))
    geo_or, gw_or = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], d["topk_weights"],
                                            grad_eo_init=np.full((cap, H), POISON_BF16, np.uint16))
    assert np.array_equal(outs[0][0], geo_or)
    _check_grad_w(outs[0][1], gw_or, gy, eo, s2r, valid)
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_backward_edges_and_rejections():
    import combine_ep_layout_amd as ep
    say("[backward] edges and rejections")
    lib = ep.library()
    # all slots masked: grad_w zero, grad_x +0, no row written
    cfg = Config("edge", 40, 256, 3, 5, 5, 8)
    d = generate(cfg, 0)
    d["topk_idx"] = np.full((40, 3), -1, np.int32)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    cap = h.capacity_rows
    eo = torch.randn(cap, 256, device=dev()).to(torch.bfloat16)
    gy = torch.randn(40, 256, device=dev()).to(torch.bfloat16)
    geo = torch.full((cap, 256), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    _, gw = h.combine_backward(epoch, gy, eo, geo)
    gx = h.dispatch_backward(epoch, eo)
    assert (gw == 0).all() and (bits_of(gx) == 0).all()
    assert (bits_of(geo) == POISON_BF16).all()
    # stale epoch, bad hidden, misaligned pointers
    P = lambda t: t.data_ptr()
    assert lib.ep_combine_backward(h.raw, epoch + 1, P(gy), P(eo), 256, P(geo), P(gw), None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_dispatch_backward(h.raw, epoch + 1, P(eo), 256, P(gx), None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_combine_backward(h.raw, epoch, P(gy), P(eo), 252, P(geo), P(gw), None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch_backward(h.raw, epoch, P(eo) + 4, 256, P(gx), None) == ep.EP_ERR_INVALID_ARGUMENT
    # rejected while a borrowed view is out
    h.borrow(to_dev_bf16(d["x"]))
    assert lib.ep_combine_backward(h.raw, epoch, P(gy), P(eo), 256, P(geo), P(gw), None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_dispatch_backward(h.raw, epoch, P(eo), 256, P(gx), None) == ep.EP_ERR_HANDLE_STATE
    h.release()
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    h.close()
    # zero tokens
    cfg0 = Config("edge0", 0, 128, 2, 4, 4, 8)
    d0 = generate(cfg0, 0)
    h0 = new_handle(cfg0, max_tokens=8)
    e0 = h0.layout(*device_routing(d0))
    h0.combine_backward(e0, torch.empty(0, 128, dtype=torch.bfloat16, device=dev()),
                        torch.zeros(h0.capacity_rows, 128, dtype=torch.bfloat16, device=dev()))
    h0.dispatch_backward(e0, torch.zeros(h0.capacity_rows, 128, dtype=torch.bfloat16, device=dev()))
    torch.cuda.synchronize()
    h0.close()
