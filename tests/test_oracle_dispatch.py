"""Pins for the oracle's dispatch (CPU only).

bf16 dispatch: every real pool row is a bitwise copy of its source token's row
(StreamEP README, "Streaming dispatch in one paragraph": each landed
(token, k) pair is written into its pool slot).  FP8 dispatch stores the same
token's e4m3fn codes and UE8M0 scales in each of its rows (instagit page, "FP8
and Quantization Support").  Pins: the closed form pool[r] == x[recv[r]]
computed with numpy fancy indexing; padding rows untouched; FP8 rows equal the
pinned per-row quantiser and agree with torch's float8 cast.
"""
import numpy as np
import torch

import oracle
from synth import CONFIGS, generate, bf16_to_f32


def test_bf16_closed_form_and_padding_untouched():
    cfg = CONFIGS["tiny"]
    d = generate(cfg, 0)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    recv = L["pool_recv_token"]
    init = np.full((L["capacity_rows"], cfg.hidden), 0xBEEF, np.uint16)
    pool = oracle.dispatch_bf16(d["x"], recv, pool_init=init)
    real = recv >= 0
    assert np.array_equal(pool[real], d["x"][recv[real]])
    assert (pool[~real] == 0xBEEF).all()


def test_fp8_rows_match_torch_cast():
    cfg = CONFIGS["decode"].replace(tokens=64)
    d = generate(cfg, 0)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    recv = L["pool_recv_token"]
    cap, H = L["capacity_rows"], cfg.hidden
    pool, scales = oracle.dispatch_fp8(d["x"], recv,
                                       pool_init=np.full((cap, H), 0xAA, np.uint8),
                                       scales_init=np.full((cap, H // 128), 0x55, np.uint8))
    real = recv >= 0
    assert (pool[~real] == 0xAA).all() and (scales[~real] == 0x55).all()
    # every row of a token carries the same bytes
    for t in range(cfg.tokens):
        rows = np.flatnonzero(recv == t)
        assert len(rows) == cfg.top_k
        assert (pool[rows] == pool[rows[0]]).all() and (scales[rows] == scales[rows[0]]).all()
        # torch's cast of x / 2^e gives the same codes (|x / 2^e| <= 448 by the scale rule)
        xf = bf16_to_f32(d["x"][t]).reshape(-1, 128).astype(np.float64)
        e = scales[rows[0]].astype(np.int64) - 127
        v = (xf * 2.0 ** (-e[:, None])).astype(np.float32).ravel()
        want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(pool[rows[0]], want)
