"""Shared helpers of the GPU parity tests: device copies of the seeded inputs,
the oracle's results for them (cached per workload), and bf16 ulp distance."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from synth import CONFIGS, Config, generate, bf16_to_f32


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda", 0)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def ord_bf16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_bf16(a) - ord_bf16(b))


@functools.lru_cache(maxsize=4)
def inputs(name: str, tokens: int = -1, seed: int = 0):
    cfg = CONFIGS[name]
    if tokens >= 0:
        cfg = cfg.replace(tokens=tokens)
    d = generate(cfg, seed)
    return cfg, d


@functools.lru_cache(maxsize=4)
def oracle_layout(name: str, tokens: int = -1, seed: int = 0):
    cfg, d = inputs(name, tokens, seed)
    return oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)


def new_handle(cfg: Config, max_tokens: int = -1):
    import combine_ep_layout_amd as ep
    return ep.EpHandle(cfg.tokens if max_tokens < 0 else max_tokens, cfg.top_k,
                       cfg.num_experts, cfg.block_m)


def device_routing(d):
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    return idx, w


LAYOUT_ARRAYS = ["expert_counts", "expert_pool_block_offset", "tile_expert",
                 "pool_arrival_target", "slot_to_pool_row", "pool_recv_token"]


def compare_layout(h, L) -> None:
    for name in LAYOUT_ARRAYS:
        got = h.array(name).cpu().numpy()
        want = L[name]
        assert got.shape == want.shape, (name, got.shape, want.shape)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[:8]}: "
                                 f"got {got[bad[:8]]}, want {want[bad[:8]]}")
    assert int(h.array("num_tiles").cpu()[0]) == L["num_tiles"]
    nt = L["num_tiles"]
    assert (h.array("pool_arrival_count").cpu().numpy()[:nt] == 0).all()


POISON_BF16 = 0xBEEF
POISON_U8 = 0xA5


def full_path_check(cfg: Config, d, fp8: bool = False, tile_ready: bool = False,
                    max_tokens: int = -1):
    """Run layout, dispatch and combine on the GPU for inputs d and compare
    every output with the oracle: layout arrays and pool bytes bit-exact,
    padding rows untouched, combine within one bf16 ulp (returns the count
    of non-identical combine elements)."""
    import combine_ep_layout_amd as ep
    from synth import expert_rows
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m,
                      cap=None if max_tokens < 0 else
                      oracle.capacity_rows(max_tokens, K, cfg.num_experts, cfg.block_m))
    h = new_handle(cfg, max_tokens)
    idx, w = device_routing(d)
    epoch = h.layout(idx, w)
    compare_layout(h, L)
    x = to_dev_bf16(d["x"])
    cap = h.capacity_rows
    recv = L["pool_recv_token"]
    real = recv >= 0
    if fp8:
        pool = torch.full((cap, H), POISON_U8, dtype=torch.uint8, device=dev())
        scales = torch.full((cap, H // 128), POISON_U8, dtype=torch.uint8, device=dev())
        h.dispatch(x, pool, scales, fp8=True, tile_ready=tile_ready)
        op, osc = oracle.dispatch_fp8(d["x"], recv,
                                      pool_init=np.full((cap, H), POISON_U8, np.uint8),
                                      scales_init=np.full((cap, H // 128), POISON_U8, np.uint8))
        assert np.array_equal(pool.cpu().numpy(), op)
        assert np.array_equal(scales.cpu().numpy(), osc)
    else:
        pool = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16,
                          device=dev()).view(torch.bfloat16)
        h.dispatch(x, pool, None, tile_ready=tile_ready)
        op = oracle.dispatch_bf16(d["x"], recv,
                                  pool_init=np.full((cap, H), POISON_BF16, np.uint16))
        assert np.array_equal(bits_of(pool), op)
    # combine on seeded expert rows; padding rows hold NaN and must never be read
    o_slot = expert_rows(T, K, H, seed=5)
    eo = np.full((cap, H), 0x7FC0, np.uint16)
    s2r = L["slot_to_pool_row"].reshape(T, K)
    valid = s2r >= 0
    eo[s2r[valid]] = o_slot[valid]
    y = h.combine(epoch, to_dev_bf16(eo))
    y_or = oracle.combine(eo, L["slot_to_pool_row"], d["topk_weights"])
    got = bits_of(y)
    assert got.shape == y_or.shape
    diff = ulp_diff(got, y_or)
    assert diff.max(initial=0) <= 1
    assert h.sync_status() == (ep.EP_ERR_BAD_ROUTING if L["error"] else ep.EP_OK)
    h.close()
    return int((diff > 0).sum())
