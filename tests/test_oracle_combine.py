"""Pins for the oracle's combine and bf16 rounding (CPU only).

Combine is the routing-weighted sum y_t = sum_j p_{t,j} o_{t,j} back in
original token order (blog "DeepEP MoE dispatch/combine", section on router
weights; instagit page, "Low-Latency Combine Kernel").  Pins: hand-worked
cases; torch's float32 -> bfloat16 cast (library routine) for the final
rounding; a float64 dense reference within the recursive-summation error
bound (Higham, Accuracy and Stability of Numerical Algorithms, sec. 4.2:
|fl(sum) - sum| <= gamma_{n-1} sum |terms| with gamma_n = n u / (1 - n u));
closed forms: identity experts with weights summing to one return x
bit-exactly, and the tiny workload's scaled experts give x * sum_k w_k (e_k+1)/8.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate, expert_rows, bf16_from_f32, bf16_to_f32
from conftest import parse_golden


def test_golden_hand_worked(golden_dir):
    cases = parse_golden(os.path.join(golden_dir, "combine_hand.txt"))
    assert len(cases) >= 6
    for case in cases:
        wtxt = case["weights"].split()
        K = len(wtxt)
        rows = [[float(v) for v in part.split()] for part in case["rows"].split("|")]
        H = len(rows[0])
        eo = bf16_from_f32(np.array(rows, np.float32))
        valid = np.array([w != "x" for w in wtxt])
        w = np.array([[0.0 if v == "x" else float(v) for v in wtxt]], np.float32)
        s2r = np.where(valid, np.arange(K), -1).astype(np.int32)
        y = oracle.combine(eo, s2r, w)
        want = bf16_from_f32(np.array([float(v) for v in case["y"].split()], np.float32))
        assert y.shape == (1, H)
        assert np.array_equal(y[0], want), case["case"]
        # the gathered form agrees
        y2 = oracle.combine_gathered(eo[None, :, :], valid[None, :], w)
        assert np.array_equal(y2[0], want)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around every 16-bit boundary
    hi = rng.integers(0, 1 << 16, 4096, dtype=np.uint32) << 16
    u = np.concatenate([u, hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi])
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    got = oracle.f32_to_bf16_n(f)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert oracle.f32_to_bf16(float("nan")) == 0x7FC0
    assert oracle.bf16_to_f32(0x3F80) == 1.0 and oracle.bf16_to_f32(0xC000) == -2.0


def _ord(b):
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


@pytest.mark.parametrize("name", ["tiny", "decode", "share"])
def test_against_float64_within_summation_bound(name):
    cfg = CONFIGS[name]
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    if name == "share":
        T = 1024
        d = {k: v[:T] for k, v in d.items()}
        H = 3072
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    o_slot = expert_rows(T, K, H, seed=0)
    eo = np.full((L["capacity_rows"], H), 0x7FC0, np.uint16)   # padding is NaN
    s2r = L["slot_to_pool_row"].reshape(T, K)
    valid = s2r >= 0
    eo[s2r[valid]] = o_slot[valid]
    w = d["topk_weights"]
    y = oracle.combine(eo, L["slot_to_pool_row"], w)
    assert not np.isnan(bf16_to_f32(y)).any()
    # float64 reference: each product w * o is exact in float64
    of = bf16_to_f32(o_slot).astype(np.float64)
    terms = np.where(valid[:, :, None], w.astype(np.float64)[:, :, None] * of, 0.0)
    ystar = terms.sum(axis=1)
    absum = np.abs(terms).sum(axis=1)
    u = 2.0 ** -24
    gam = (K * u) / (1 - K * u)
    yo = bf16_to_f32(y).astype(np.float64)
    # accumulation error plus one bf16 rounding (half an ulp, relative 2^-8)
    bound = gam * absum + 2.0 ** -8 * (np.abs(ystar) + gam * absum) + 1e-45
    assert np.all(np.abs(yo - ystar) <= bound)
    # where the fp32 chain's error bound is below a quarter bf16 ulp of the result,
    # rounding the exact sum directly can differ from it by at most one ulp, and rarely
    yexact = bf16_from_f32(ystar.astype(np.float32))
    diff = np.abs(_ord(yexact) - _ord(y))
    well = gam * absum <= 2.0 ** -10 * np.abs(ystar)
    assert well.mean() > 0.9
    assert diff[well].max() <= 1 and (diff > 0).mean() < 0.01


@pytest.mark.parametrize("name", ["tiny", "decode", "share", "stream"])
def test_identity_experts_return_x(name):
    cfg = CONFIGS[name]
    if name == "stream":
        cfg = cfg.replace(tokens=2048, hidden=512)
    d = generate(cfg, 0)
    T, K = cfg.tokens, cfg.top_k
    idx = d["topk_idx"]
    L = oracle.layout(idx, cfg.num_experts, cfg.block_m)
    pool = oracle.dispatch_bf16(d["x"], L["pool_recv_token"])
    valid = idx >= 0
    # renormalise the weights over the unmasked slots (test only)
    w64 = np.where(valid, d["topk_weights"].astype(np.float64), 0.0)
    tot = w64.sum(1, keepdims=True)
    w = np.where(tot > 0, w64 / np.where(tot > 0, tot, 1), 0.0).astype(np.float32)
    y = oracle.combine(pool, L["slot_to_pool_row"], w)
    has = valid.any(1)
    # the accumulator starts at +0, so an input -0 comes back as +0 (+0 + -0 = +0)
    xs = np.where(d["x"] == 0x8000, 0, d["x"])
    assert np.array_equal(y[has], xs[has])
    assert (y[~has] == 0).all()


def test_tiny_scaled_experts_closed_form():
    cfg = CONFIGS["tiny"]
    d = generate(cfg, 0)
    idx, w = d["topk_idx"], d["topk_weights"]
    L = oracle.layout(idx, cfg.num_experts, cfg.block_m)
    pool = oracle.dispatch_bf16(d["x"], L["pool_recv_token"])
    recv = L["pool_recv_token"]
    te = L["tile_expert"]
    rows = np.flatnonzero(recv >= 0)
    scale = (te[rows // cfg.block_m] + 1) / 8.0
    eo = np.zeros_like(pool)
    eo[rows] = bf16_from_f32(bf16_to_f32(pool[rows]) * scale[:, None].astype(np.float32))
    y = oracle.combine(eo, L["slot_to_pool_row"], w)
    xf = bf16_to_f32(d["x"]).astype(np.float64)
    factor = (w.astype(np.float64) * (idx + 1) / 8.0).sum(1)
    want = xf * factor[:, None]
    got = bf16_to_f32(y).astype(np.float64)
    # each scaled row is exact before its bf16 rounding (<= 1/2 ulp), the sum adds <= 1/2 ulp
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    assert np.all(np.abs(got - want) <= 2 * ulp + 1e-30)


def test_single_slot_weight_one_is_copy_and_zero_weight_is_zero():
    rng = np.random.default_rng(1)
    o = bf16_from_f32(rng.standard_normal((3, 64), dtype=np.float32))
    s2r = np.array([2, 0, 1], np.int32)
    y = oracle.combine(o, s2r, np.ones((3, 1), np.float32))
    assert np.array_equal(y, o[[2, 0, 1]])
    y0 = oracle.combine(o, s2r, np.zeros((3, 1), np.float32))
    assert np.array_equal(bf16_to_f32(y0), np.zeros((3, 64), np.float32))
    yh = oracle.combine(o, s2r, np.full((3, 1), 0.5, np.float32))
    assert np.array_equal(bf16_to_f32(yh), bf16_to_f32(o[[2, 0, 1]]) * np.float32(0.5))


def test_nan_rounds_to_the_quiet_nan_with_its_sign():
    """NaN of any payload rounds to the quiet NaN 0x7FC0 with its sign kept
    (reading 10's final rounding).  Patterns with low payload bits only are
    the ones a truncating conversion would turn into infinity.  (Not compared
    with torch: its vectorised CPU cast writes other NaN patterns.)"""
    pos = np.array([0x7F800001, 0x7F80FFFF, 0x7FA00000, 0x7FC00000, 0x7FFFFFFF], np.uint32)
    got = oracle.f32_to_bf16_n(np.concatenate([pos, pos | 0x80000000]).view(np.float32))
    assert np.array_equal(got[:5], np.full(5, 0x7FC0, np.uint16))
    assert np.array_equal(got[5:], np.full(5, 0xFFC0, np.uint16))


def test_fp32_fma_chain_in_ascending_slot_order():
    """Reading 10 fixes the accumulation: fp32 from +0, one fused
    multiply-add per unmasked slot in ascending k, one rounding to bf16.  Two
    hand-worked tokens sit on bf16 rounding midpoints, where any other
    accumulation rounds the other way.
    Token 0, slots (w, o) = (1 + 2^-8, 1), (1, 2^-24), (1, 2^-24): in
    ascending order each 2^-24 lands on an fp32 tie and rounds back (to even)
    to 1 + 2^-8, a bf16 tie that rounds to even: 1.0 (0x3F80).  Descending
    slots, or an exact sum, reach 1 + 2^-8 + 2^-23, which rounds up to 0x3F81.
    Token 1, slots (1, 1), (w2, 3) with w2 = 0x3AAAAB56, so that w2 * 3 =
    2^-8 + 2^-24 + 2^-32 exactly: the fused step rounds 1 + w2 * 3 once, up
    to 1 + 2^-8 + 2^-23: 0x3F81.  A separate multiply first rounds the product
    to 2^-8 + 2^-24 (an fp32 tie, to even), and the add then ties to even at
    1 + 2^-8: 0x3F80."""
    w2 = float(np.array([0x3AAAAB56], np.uint32).view(np.float32)[0])
    assert Fraction(w2) * 3 == Fraction(1, 2**8) + Fraction(1, 2**24) + Fraction(1, 2**32)
    H = 8
    # rows: 1.0, 2^-24, 2^-24, 1.0, 3.0 as bf16 patterns
    eo = np.repeat(np.array([0x3F80, 0x3380, 0x3380, 0x3F80, 0x4040], np.uint16)[:, None], H, 1)
    s2r = np.array([0, 1, 2, 3, 4, -1], np.int32)
    w = np.array([[1 + 2.0 ** -8, 1.0, 1.0], [1.0, w2, 0.0]], np.float32)
    assert float(w[0, 0]) == 1 + 2.0 ** -8 and float(w[1, 1]) == w2
    y = oracle.combine(eo, s2r, w)
    assert np.array_equal(y, np.array([[0x3F80] * H, [0x3F81] * H], np.uint16))
    valid = (s2r >= 0).reshape(2, 3)
    y2 = oracle.combine_gathered(eo[np.where(s2r >= 0, s2r, 0)].reshape(2, 3, H), valid, w)
    assert np.array_equal(y2, y)


def test_gathered_combine_skips_masked_slots():
    """A masked slot takes no part even when its gathered row is NaN and its
    weight is not zero: y = bf16(1 * x) = x."""
    rng = np.random.default_rng(3)
    x = bf16_from_f32(rng.standard_normal(64, dtype=np.float32))
    rows = np.stack([x, np.full(64, 0x7FC0, np.uint16)])[None]
    y = oracle.combine_gathered(rows, np.array([[True, False]]), np.array([[1.0, 0.5]], np.float32))
    assert np.array_equal(y[0], x)
