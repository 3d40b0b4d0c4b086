"""Edge cases of the routing and of the C ABI on the GPU (blog "DeepEP MoE
dispatch/combine", section on extreme routing: all assignments on one expert,
an expert with zero rows, counts that are and are not multiples of the
alignment, top-1 / top-2 / the model's top-k, several experts of one token
together, FP8 dispatch with BF16 combine, and misuse of a stale handle)."""
import numpy as np
import pytest
import torch

import oracle
from synth import Config, generate
from gpu_helpers import say, full_path_check, new_handle, device_routing, to_dev_bf16, dev

pytestmark = pytest.mark.gpu


def _custom(T, K, E, BM, H, idx=None, seed=0, fp8=False):
    cfg = Config("edge", T, H, K, E, E, BM)
    d = generate(cfg, seed)
    if idx is not None:
        d["topk_idx"] = np.ascontiguousarray(np.asarray(idx, np.int32).reshape(T, K))
    return cfg, d


@pytest.mark.parametrize("fp8", [False, True])
def test_zero_tokens(fp8):
    say(f"[edge] T=0 fp8={fp8}")
    cfg, d = _custom(0, 4, 5, 8, 256)
    full_path_check(cfg, d, fp8=fp8, max_tokens=16)


def test_one_token():
    say("[edge] T=1")
    cfg, d = _custom(1, 8, 16, 4, 256)
    full_path_check(cfg, d, fp8=True)


@pytest.mark.parametrize("BM", [1, 7, 64, 128])
def test_all_slots_one_expert(BM):
    say(f"[edge] all slots on one expert, BM={BM}")
    T, K = 700, 1
    cfg, d = _custom(T, K, 9, BM, 128, idx=np.full(T * K, 6))
    full_path_check(cfg, d)


def test_all_masked():
    say("[edge] all slots masked")
    cfg, d = _custom(50, 3, 4, 16, 256, idx=np.full(150, -1))
    full_path_check(cfg, d, fp8=True)


def test_exact_multiples_of_block_m():
    say("[edge] counts exact multiples of BLOCK_M")
    T, K, E, BM = 64, 2, 4, 8
    idx = np.repeat(np.arange(E), T * K // E)          # 32 slots per expert, sorted by slot
    cfg, d = _custom(T, K, E, BM, 128, idx=idx)
    full_path_check(cfg, d)


@pytest.mark.parametrize("K", [1, 2, 3, 8, 16, 32])
def test_top_k_values(K):
    say(f"[edge] top_k={K}")
    cfg, d = _custom(97, K, 33, 5, 384, seed=K)
    full_path_check(cfg, d, fp8=True)


def test_duplicate_experts_in_one_token():
    say("[edge] duplicate experts within a token")
    rng = np.random.default_rng(4)
    T, K, E = 200, 4, 3
    idx = rng.integers(-1, E, size=(T, K))
    cfg, d = _custom(T, K, E, 16, 128, idx=idx)
    full_path_check(cfg, d)


def test_out_of_range_ids_flagged_and_masked():
    import combine_ep_layout_amd as ep
    say("[edge] ids outside [-1, E)")
    rng = np.random.default_rng(8)
    T, K, E = 300, 2, 6
    idx = rng.integers(-1, E, size=(T, K))
    idx[5, 0], idx[17, 1], idx[250, 0] = 6, -2, 1000
    cfg, d = _custom(T, K, E, 8, 128, idx=idx)
    full_path_check(cfg, d)                 # also checks EP_ERR_BAD_ROUTING is reported
    # multi-workgroup layout path (more than 16384 slots)
    T = 10000
    idx = rng.integers(-1, E, size=(T, K))
    idx[9999, 1] = 7
    cfg, d = _custom(T, K, E, 8, 128, idx=idx)
    full_path_check(cfg, d)


def test_single_expert_block_m_one():
    say("[edge] E=1, BM=1")
    idx = np.random.default_rng(6).integers(-1, 1, size=(33, 2))    # expert 0 twice, or masked
    cfg, d = _custom(33, 2, 1, 1, 128, idx=idx)
    full_path_check(cfg, d, fp8=True)


def test_fewer_tokens_than_capacity():
    say("[edge] num_tokens below max_tokens")
    cfg, d = _custom(100, 8, 64, 64, 512, seed=3)
    full_path_check(cfg, d, fp8=True, max_tokens=256)


def test_abi_rejections():
    import combine_ep_layout_amd as ep
    say("[edge] ABI rejections")
    lib = ep.library()
    cfg, d = _custom(32, 2, 4, 8, 256)
    h = new_handle(cfg)
    H = 256
    x = to_dev_bf16(d["x"])
    pool, _ = h.new_pool(H)
    fpool, fscales = h.new_pool(H, fp8=True)
    y = torch.empty(32, H, dtype=torch.bfloat16, device=dev())
    raw = h.raw
    P = lambda t: None if t is None else t.data_ptr()
    # dispatch / combine before any layout
    assert lib.ep_dispatch(raw, P(x), H, P(pool), None, 0, None, None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_combine(raw, 0, P(pool), H, P(y), None) == ep.EP_ERR_HANDLE_STATE
    idx, w = device_routing(d)
    # too many tokens
    assert lib.ep_layout(raw, P(idx), P(w), 33, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_layout(raw, P(idx), P(w), -1, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_layout(raw, None, P(w), 32, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    epoch = h.layout(idx, w)
    # stale or future epoch
    assert lib.ep_combine(raw, epoch + 1, P(pool), H, P(y), None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_combine(raw, epoch - 1, P(pool), H, P(y), None) == ep.EP_ERR_HANDLE_STATE
    # hidden not a multiple of 8; FP8 hidden not a multiple of 128
    assert lib.ep_dispatch(raw, P(x), 250, P(pool), None, 0, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_combine(raw, epoch, P(pool), 0, P(y), None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(raw, P(x), 200, P(fpool), P(fscales), ep.EP_DISPATCH_FP8, None,
                           None) == ep.EP_ERR_INVALID_ARGUMENT
    # FP8 without scales, scales without FP8, unknown flag bits
    assert lib.ep_dispatch(raw, P(x), H, P(fpool), None, ep.EP_DISPATCH_FP8, None,
                           None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(raw, P(x), H, P(pool), P(fscales), 0, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(raw, P(x), H, P(pool), None, 1 << 7, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    # pointers that are not 16-byte aligned
    assert lib.ep_dispatch(raw, P(x) + 2, H, P(pool), None, 0, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_combine(raw, epoch, P(pool) + 8, H, P(y), None) == ep.EP_ERR_INVALID_ARGUMENT
    # a rejected call left the handle usable, and the valid epoch still works
    torch.cuda.synchronize()
    h.dispatch(x, pool)
    h.combine(epoch, pool, y)
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    # a new layout invalidates the old epoch
    epoch2 = h.layout(idx, w)
    assert epoch2 == epoch + 1
    assert lib.ep_combine(raw, epoch, P(pool), H, P(y), None) == ep.EP_ERR_HANDLE_STATE
    h.close()
