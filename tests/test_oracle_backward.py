"""Pins for the oracle's backward functions (CPU only).

combine_grads / dispatch_grads are named by the StreamEP README ("What's in
the box"); their values are the derivatives of the forward definitions.
Pins: hand-worked cases; numpy float64 dot products and sums (library
routines) within the rounding bounds of the stated arithmetic; torch's
float32 -> bfloat16 cast for the gradient rows; the adjoint identities
<combine(o), g> = <o, combine^T(g)> and <dispatch(x), gp> = <x, dispatch^T(gp)>.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate, expert_rows, bf16_from_f32, bf16_to_f32
from conftest import parse_golden


def _floats(s):
    return [float(v) for v in s.split()]


def test_golden_hand_worked(golden_dir):
    cases = parse_golden(os.path.join(golden_dir, "backward_hand.txt"))
    assert len(cases) >= 6
    for case in cases:
        if "weights" in case:
            wt = case["weights"].split()
            K = len(wt)
            valid = np.array([v != "x" for v in wt])
            w = np.array([[0.0 if v == "x" else float(v) for v in wt]], np.float32)
            gy = bf16_from_f32(np.array([_floats(case["grad_y"])], np.float32))
            rows = bf16_from_f32(np.array([_floats(r) for r in case["rows"].split("|")], np.float32))
            s2r = np.where(valid, np.arange(K), -1).astype(np.int32)
            poison = np.full_like(rows, 0xBEEF)
            geo, gw = oracle.combine_backward(gy, rows, s2r, w, grad_eo_init=poison)
            for k, part in enumerate(case["grad_rows"].split("|")):
                if part.strip() == "-":
                    assert (geo[k] == 0xBEEF).all(), case["case"]
                else:
                    want = bf16_from_f32(np.array(_floats(part), np.float32))
                    assert np.array_equal(geo[k], want), case["case"]
            assert np.array_equal(gw[0], np.array(_floats(case["grad_w"]), np.float32)), case["case"]
        else:
            slot_rows = [[int(v) for v in p.split()] for p in case["slot_rows"].split("|")]
            T, K = len(slot_rows), len(slot_rows[0])
            gp = bf16_from_f32(np.array([_floats(r) for r in case["grad_pool"].split("|")], np.float32))
            gx = oracle.dispatch_backward(gp, np.array(slot_rows, np.int32).ravel(), T, K)
            want = bf16_from_f32(np.array([_floats(r) for r in case["grad_x"].split("|")], np.float32))
            assert np.array_equal(gx, want), case["case"]


def _setup(name, tokens=None, seed=0):
    cfg = CONFIGS[name]
    if tokens is not None:
        cfg = cfg.replace(tokens=tokens)
    d = generate(cfg, seed)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    o_slot = expert_rows(T, K, H, seed=3)
    eo = np.full((L["capacity_rows"], H), 0x7FC0, np.uint16)
    s2r = L["slot_to_pool_row"].reshape(T, K)
    valid = s2r >= 0
    eo[s2r[valid]] = o_slot[valid]
    gy = expert_rows(T, 1, H, seed=4)[:, 0, :]
    return cfg, d, L, eo, gy, s2r, valid


@pytest.mark.parametrize("name,tokens", [("tiny", None), ("decode", 64), ("share", 512)])
def test_combine_backward_against_numpy(name, tokens):
    cfg, d, L, eo, gy, s2r, valid = _setup(name, tokens)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    w = d["topk_weights"]
    poison = np.full_like(eo, 0xBEEF)
    geo, gw = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], w, grad_eo_init=poison)
    g64 = bf16_to_f32(gy).astype(np.float64)
    for t in range(T):
        for k in range(K):
            if not valid[t, k]:
                assert gw[t, k] == 0.0
                continue
            r = s2r[t, k]
            o64 = bf16_to_f32(eo[r]).astype(np.float64)
            prod = g64[t] * o64
            exact = np.dot(g64[t], o64)                       # numpy float64 dot
            bound = np.spacing(np.float32(abs(exact))) + 2 * H * 2.0 ** -53 * np.abs(prod).sum()
            assert abs(float(gw[t, k]) - exact) <= bound, (t, k)
            # gradient rows: fp32 product rounded by torch to bf16
            want = torch.from_numpy(np.float32(w[t, k]) * bf16_to_f32(gy[t])).to(torch.bfloat16)
            assert np.array_equal(geo[r], want.view(torch.int16).numpy().view(np.uint16))
    # rows that belong to no slot are never written
    assert (geo[L["pool_recv_token"] < 0] == 0xBEEF).all()


@pytest.mark.parametrize("name,tokens", [("decode", 128), ("share", 1024), ("stream", 256)])
def test_dispatch_backward_against_numpy(name, tokens):
    cfg, d, L, eo, gy, s2r, valid = _setup(name, tokens)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    gp = eo                                                # any rows: padding must not be read
    gx = oracle.dispatch_backward(gp, L["slot_to_pool_row"], T, K)
    assert not np.isnan(bf16_to_f32(gx)).any()
    rows = np.where(valid, s2r, 0)
    terms = np.where(valid[:, :, None], bf16_to_f32(gp[rows]).astype(np.float64), 0.0)
    exact = terms.sum(1)
    absum = np.abs(terms).sum(1)
    u = 2.0 ** -24
    gam = K * u / (1 - K * u)
    got = bf16_to_f32(gx).astype(np.float64)
    assert np.all(np.abs(got - exact) <= gam * absum + 2.0 ** -8 * (np.abs(exact) + gam * absum) + 1e-45)
    one = valid.sum(1) == 1
    kk = valid.argmax(1)
    single = gp[s2r[np.arange(T), kk]]
    assert np.array_equal(np.where(single == 0x8000, 0, single)[one], gx[one])
    assert (gx[valid.sum(1) == 0] == 0).all()


@pytest.mark.parametrize("name,tokens", [("tiny", None), ("share", 512)])
def test_adjoint_identities(name, tokens):
    cfg, d, L, eo, gy, s2r, valid = _setup(name, tokens)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    w = d["topk_weights"]
    real = L["pool_recv_token"] >= 0
    # combine: <combine(o), g> = <o, combine^T(g)> over the real rows
    y = oracle.combine(eo, L["slot_to_pool_row"], w)
    geo, _ = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], w)
    lhs = (bf16_to_f32(y).astype(np.float64) * bf16_to_f32(gy)).sum()
    rhs = (bf16_to_f32(eo[real]).astype(np.float64) * bf16_to_f32(geo[real])).sum()
    scale = np.abs(bf16_to_f32(eo[real]).astype(np.float64)).sum() * np.abs(bf16_to_f32(gy)).max()
    assert abs(lhs - rhs) <= 2.0 ** -7 * scale
    # dispatch: <dispatch(x), gp> = <x, dispatch^T(gp)>
    pool = oracle.dispatch_bf16(d["x"], L["pool_recv_token"])
    gp = np.where(real[:, None], eo, 0).astype(np.uint16)
    gx = oracle.dispatch_backward(gp, L["slot_to_pool_row"], T, K)
    lhs = (bf16_to_f32(pool[real]).astype(np.float64) * bf16_to_f32(gp[real])).sum()
    rhs = (bf16_to_f32(d["x"]).astype(np.float64) * bf16_to_f32(gx)).sum()
    scale = (np.abs(bf16_to_f32(pool[real])).astype(np.float64) * np.abs(bf16_to_f32(gp[real]))).sum()
    assert abs(lhs - rhs) <= 2.0 ** -7 * scale
