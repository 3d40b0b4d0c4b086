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


def _check_grad_w(got, want, gy, eo, s2r, valid):
    H = gy.shape[1]
    assert (got[~valid] == 0).all()
    g64 = bf16_to_f32(gy).astype(np.float64)
    ts, ks = np.nonzero(valid)
    o64 = bf16_to_f32(eo[s2r[ts, ks]]).astype(np.float64)
    absum = np.abs(g64[ts] * o64).sum(1)
    w = want[ts, ks].astype(np.float64)
    bound = np.spacing(np.abs(want[ts, ks])).astype(np.float64) + 2 * H * 2.0 ** -53 * absum
    diff = np.abs(got[ts, ks].astype(np.float64) - w)
    assert np.all(diff <= bound)
    return int((diff > 0).sum())


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


def test_backward_full_size_sampled():
    say("[backward] prefill full size, sampled tokens")
    cfg, d = inputs("prefill")
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    g = torch.Generator(device=dev())
    g.manual_seed(77)
    eo = torch.randn(h.capacity_rows, H, generator=g, device=dev()).to(torch.bfloat16)
    gy = torch.randn(T, H, generator=g, device=dev()).to(torch.bfloat16)
    geo, gw = h.combine_backward(epoch, gy, eo)
    gx = h.dispatch_backward(epoch, eo)
    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(T, size=256, replace=False))
    s2r = L["slot_to_pool_row"].reshape(T, K)
    w = d["topk_weights"]
    gy_h = bits_of(gy[torch.from_numpy(toks).to(dev())])
    for i, t in enumerate(toks):
        rows = s2r[t]
        vr = rows[rows >= 0]
        eo_rows = bits_of(eo[torch.from_numpy(vr.astype(np.int64)).to(dev())])
        # single-token oracle calls on gathered rows
        sub_s2r = np.where(rows >= 0, np.cumsum(rows >= 0) - 1, -1).astype(np.int32)
        geo_or, gw_or = oracle.combine_backward(gy_h[i:i + 1], eo_rows, sub_s2r, w[t:t + 1])
        assert np.array_equal(bits_of(geo[torch.from_numpy(vr.astype(np.int64)).to(dev())]), geo_or)
        _check_grad_w(gw[t:t + 1].cpu().numpy(), gw_or, gy_h[i:i + 1], eo_rows,
                      sub_s2r.reshape(1, K), (rows >= 0).reshape(1, K))
        gx_or = oracle.dispatch_backward(eo_rows, sub_s2r, 1, K)
        assert np.array_equal(bits_of(gx[t:t + 1]), gx_or)
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
