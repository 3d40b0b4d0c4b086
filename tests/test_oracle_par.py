"""The threaded oracle front end used by the full-size GPU parity tests
returns exactly what the oracle's own functions return on the whole batch."""
import numpy as np
import pytest

import oracle
from oracle import par as oracle_par
from synth import CONFIGS, generate, expert_rows


@pytest.mark.parametrize("name,tokens", [("decode", -1), ("stream", 300), ("tiny", -1)])
def test_threaded_front_end_equals_oracle(name, tokens):
    cfg = CONFIGS[name]
    if tokens >= 0:
        cfg = cfg.replace(tokens=tokens)
    cfg = cfg.replace(hidden=512)
    d = generate(cfg, 3)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    recv = L["pool_recv_token"]
    real = recv >= 0
    for kind in ("ue8m0", "f32", "pow2_f32"):
        q, s = oracle_par.quantize_tokens(d["x"], kind=kind)
        op, osc = oracle.dispatch_fp8_scaled(d["x"], recv, kind)
        assert np.array_equal(op[real], q[recv[real]]), kind
        assert np.array_equal(osc[real], s[recv[real]]), kind
    q, s = oracle_par.quantize_tokens(d["x"])
    assert np.array_equal(oracle_par.dequant_tokens(q, s), oracle.dequant_rows(q, s))
    o = expert_rows(T, K, H, seed=5)
    eo = np.full((L["capacity_rows"], H), 0x7FC0, np.uint16)
    s2r = L["slot_to_pool_row"].reshape(T, K)
    v = s2r >= 0
    eo[s2r[v]] = o[v]
    w = d["topk_weights"]
    assert np.array_equal(oracle_par.combine(eo, L["slot_to_pool_row"], w),
                          oracle.combine(eo, L["slot_to_pool_row"], w))
    gy = expert_rows(T, 1, H, seed=9)[:, 0, :]
    g1, w1 = oracle.combine_backward(gy, eo, L["slot_to_pool_row"], w,
                                     grad_eo_init=np.full_like(eo, 0xBEEF))
    g2, w2 = oracle_par.combine_backward(gy, eo, L["slot_to_pool_row"], w, np.full_like(eo, 0xBEEF))
    assert np.array_equal(g1, g2) and np.array_equal(w1, w2)
    assert np.array_equal(oracle_par.dispatch_backward(eo, L["slot_to_pool_row"], T, K),
                          oracle.dispatch_backward(eo, L["slot_to_pool_row"], T, K))
