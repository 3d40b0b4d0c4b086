"""GPU parity of combine against the oracle: y within one bf16 ulp of the
oracle's fp32 fma chain (expected bit-exact), padding rows never read, and the
end-to-end closed forms (blog "DeepEP MoE dispatch/combine", router-weight
section: y_t = sum_j p_{t,j} o_{t,j})."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate, bf16_to_f32, bf16_from_f32
from gpu_helpers import (say, inputs, oracle_layout, new_handle, device_routing, to_dev_bf16,
                         bits_of, ulp_diff, dev)

pytestmark = pytest.mark.gpu


def test_tiny_scaled_experts_end_to_end():
    """The tiny workload's experts multiply each row by (e+1)/8."""
    say("[combine] tiny, expert = x*(e+1)/8")
    cfg, d = inputs("tiny")
    L = oracle_layout("tiny")
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    pool, _ = h.new_pool(cfg.hidden)
    h.dispatch(x, pool)
    # the "experts" (test stand-in for the caller's GEMM), on the device with torch
    # only real rows are indexed: they all lie in tiles below num_tiles
    te = h.array("tile_expert").long()
    recv = h.array("pool_recv_token")
    real_t = torch.nonzero(recv >= 0).squeeze(1)
    scale = ((te[real_t // cfg.block_m] + 1).float() / 8.0)[:, None]
    eo = torch.full_like(pool, float("nan"))
    eo[real_t] = (pool[real_t].float() * scale).to(torch.bfloat16)
    y = h.combine(epoch, eo)
    # oracle side: the same experts applied to the oracle's pool
    op = oracle.dispatch_bf16(d["x"], L["pool_recv_token"])
    real = L["pool_recv_token"] >= 0
    ridx = np.flatnonzero(real)
    sc = ((L["tile_expert"][ridx // cfg.block_m] + 1) / 8.0).astype(np.float32)
    eo_or = np.full_like(op, 0x7FC0)
    eo_or[ridx] = bf16_from_f32(bf16_to_f32(op[ridx]) * sc[:, None])
    assert np.array_equal(bits_of(eo)[real], eo_or[real])
    y_or = oracle.combine(eo_or, L["slot_to_pool_row"], d["topk_weights"])
    diff = ulp_diff(bits_of(y), y_or)
    say(f"  non-identical elements: {(diff > 0).sum()}")
    assert diff.max() <= 1
    h.close()


@pytest.mark.parametrize("name", ["decode", "share"])
def test_combine_full_compare(name):
    from gpu_helpers import full_path_check
    say(f"[combine] {name} full compare")
    cfg, d = inputs(name)
    n = full_path_check(cfg.replace(fp8=False), d)
    say(f"  non-identical elements: {n}")


@pytest.mark.parametrize("name", ["prefill", "stream"])
def test_combine_full_size(name):
    """The metric's workload and the streaming one at full size: every
    element of y against the oracle's combine of the same expert rows."""
    from oracle import par as oracle_par
    say(f"[combine] {name} full size, every token")
    cfg, d = inputs(name)
    L = oracle_layout(name)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    cap, H, T = h.capacity_rows, cfg.hidden, cfg.tokens
    g = torch.Generator(device=dev())
    g.manual_seed(1234)
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    for r0 in range(0, cap, 16384):
        r1 = min(cap, r0 + 16384)
        eo[r0:r1] = torch.randn(r1 - r0, H, generator=g, device=dev()).to(torch.bfloat16)
    recv = torch.from_numpy(L["pool_recv_token"]).to(dev())
    eo[recv < 0] = float("nan")                   # rows no slot owns are never read
    y = h.combine(epoch, eo)
    eo_h = bits_of(eo)
    del eo
    y_or = oracle_par.combine(eo_h, L["slot_to_pool_row"], d["topk_weights"])
    diff = ulp_diff(bits_of(y), y_or)
    say(f"  non-identical elements: {(diff > 0).sum()} of {diff.size}")
    assert diff.max() <= 1
    h.close()


@pytest.mark.parametrize("name,tokens", [("share", -1), ("stream", 4096), ("prefill", 2048)])
def test_identity_experts_return_x(name, tokens):
    """combine(dispatch(x)) with identity experts and weights renormalised to
    sum to one over the unmasked slots returns x bit-exactly; tokens with no
    unmasked slot return +0."""
    say(f"[combine] identity {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    idx = d["topk_idx"]
    valid = idx >= 0
    w64 = np.where(valid, d["topk_weights"].astype(np.float64), 0.0)
    tot = w64.sum(1, keepdims=True)
    w = np.where(tot > 0, w64 / np.where(tot > 0, tot, 1), 0.0).astype(np.float32)
    h = new_handle(cfg)
    epoch = h.layout(torch.from_numpy(idx).to(dev()), torch.from_numpy(w).to(dev()))
    x = to_dev_bf16(d["x"])
    pool, _ = h.new_pool(cfg.hidden)
    h.dispatch(x, pool)
    y = bits_of(h.combine(epoch, pool))
    has = valid.any(1)
    # the accumulator starts at +0, so an input -0 comes back as +0 (+0 + -0 = +0)
    xs = np.where(d["x"] == 0x8000, 0, d["x"])
    assert np.array_equal(y[has], xs[has])
    assert (y[~has] == 0).all()
    h.close()


def test_fp8_dequant_experts_return_dequantised_x():
    """FP8 dispatch, the consumer stand-in's dequantisation as the expert, and
    combine with weights summing to one return bf16(e4m3(q) * 2^e) exactly."""
    say("[combine] fp8 dequant experts, decode")
    import combine_ep_layout_amd as ep
    cfg, d = inputs("decode")
    w = np.full_like(d["topk_weights"], 1.0 / cfg.top_k)      # 1/8: exact, sums to one
    h = new_handle(cfg)
    epoch = h.layout(torch.from_numpy(d["topk_idx"]).to(dev()), torch.from_numpy(w).to(dev()))
    x = to_dev_bf16(d["x"])
    pool, scales = h.new_pool(cfg.hidden, fp8=True)
    h.dispatch(x, pool, scales, fp8=True)
    out = torch.zeros(h.capacity_rows, cfg.hidden, dtype=torch.bfloat16, device=dev())
    h.tile_consume(0, pool, scales, cfg.hidden, out, fp8=True)   # seq 0: no wait
    y = bits_of(h.combine(epoch, out))
    want = np.stack([oracle.dequant_rows(*[a[None, :] for a in oracle.quantize_row(d["x"][t])])[0]
                     for t in range(cfg.tokens)])
    # the consumer's dequantised rows are bit-exact
    L = oracle_layout("decode")
    recv = L["pool_recv_token"]
    real = np.flatnonzero(recv >= 0)
    assert np.array_equal(bits_of(out[torch.from_numpy(real).to(dev())]), want[recv[real]])
    # combine returns them, with -0 coming back as +0 (the accumulator starts at +0)
    assert np.array_equal(y, np.where(want == 0x8000, 0, want))
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_nan_padding_is_never_read():
    say("[combine] NaN padding vs zero padding")
    cfg, d = inputs("share")
    L = oracle_layout("share")
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    g = torch.Generator(device=dev())
    g.manual_seed(9)
    eo = torch.randn(h.capacity_rows, cfg.hidden, generator=g, device=dev()).to(torch.bfloat16)
    pad = torch.from_numpy(L["pool_recv_token"] < 0).to(dev())
    eo[pad] = 0.0
    y0 = h.combine(epoch, eo).clone()
    eo[pad] = float("nan")
    y1 = h.combine(epoch, eo)
    assert not torch.isnan(y1).any()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    h.close()


@pytest.mark.parametrize("sync", [True, False])
def test_combine_after_dense_and_sparse_layouts(sync):
    """The plain combine, the dispatch backward and the combine backward take
    their launch shape from the density of the current layout (two
    workgroups per compute unit for 4 or more rows per token, full occupancy
    below), waiting for the layout kernel's report when it has not arrived;
    the results do not depend on it.  One handle alternates a dense and a
    sparse routing of the same size, with or without a synchronisation after
    each layout, and every combine, dispatch backward and combine backward is
    compared with the oracle (gradient rows bit for bit, weight gradients
    within the bound of the backward tests)."""
    say(f"[combine] alternating dense / sparse layouts on one handle, 6000 tokens, sync={sync}")
    dense = CONFIGS["stream"].replace(tokens=6000, hidden=1024, mask_frac=0.0, fp8=False,
                                      tile_ready=False)
    sparse = CONFIGS["share"].replace(tokens=6000, hidden=1024, num_experts=128, experts_global=128,
                                      local_keep=16)
    h = new_handle(dense)
    rng = np.random.default_rng(41)
    for it, cfg in enumerate([dense, sparse, dense, sparse]):
        d = generate(cfg, 50 + it)
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m, cap=h.capacity_rows)
        epoch = h.layout(*device_routing(d))
        if sync:
            torch.cuda.synchronize()
        rows = int((d["topk_idx"] >= 0).sum())
        eo = bf16_from_f32(rng.standard_normal((h.capacity_rows, cfg.hidden), dtype=np.float32))
        y = h.combine(epoch, to_dev_bf16(eo))
        y_or = oracle.combine(eo, L["slot_to_pool_row"], d["topk_weights"])
        assert ulp_diff(bits_of(y), y_or).max(initial=0) <= 1
        gx = h.dispatch_backward(epoch, to_dev_bf16(eo))
        assert np.array_equal(bits_of(gx), oracle.dispatch_backward(eo, L["slot_to_pool_row"],
                                                                      cfg.tokens, cfg.top_k))
        gy = bf16_from_f32(rng.standard_normal((cfg.tokens, cfg.hidden), dtype=np.float32))
        geo = torch.zeros((h.capacity_rows, cfg.hidden), dtype=torch.bfloat16, device=dev())
        _, gw = h.combine_backward(epoch, to_dev_bf16(gy), to_dev_bf16(eo), geo)
        geo_or, gw_or = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], d["topk_weights"],
                                                grad_eo_init=np.zeros((h.capacity_rows, cfg.hidden),
                                                                      np.uint16))
        assert np.array_equal(bits_of(geo), geo_or)
        s2r = L["slot_to_pool_row"].reshape(cfg.tokens, cfg.top_k)
        valid = s2r >= 0
        got = gw.cpu().numpy()
        assert (got[~valid] == 0).all()
        ts, ks = np.nonzero(valid)
        absum = np.abs(bf16_to_f32(gy[ts]).astype(np.float64) *
                       bf16_to_f32(eo[s2r[ts, ks]]).astype(np.float64)).sum(1)
        bound = (np.spacing(np.abs(gw_or[ts, ks])).astype(np.float64) +
                 2 * cfg.hidden * 2.0 ** -53 * absum)
        assert np.all(np.abs(got[ts, ks].astype(np.float64) - gw_or[ts, ks]) <= bound)
        say(f"  layout {it}: {rows / cfg.tokens:.2f} rows per token, combine and both backward calls match")
    assert h.sync_status() == 0
    h.close()
