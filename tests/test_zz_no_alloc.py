"""ep_layout_noalloc, the layout entry point that allocates nothing (for
callers that cannot allocate device memory): its arrays, written into buffers
the caller owns with the library's fixed scratch array as the workspace,
equal ep_layout's arrays and the oracle's bit for bit.  Two calls in a row
share the scratch array; the second has fewer tokens, so its workgroup rows
of the scratch are a prefix of the first call's and must not be mistaken for
its own."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import say, dev, device_routing, new_handle, LAYOUT_ARRAYS
from synth import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _noalloc_layout(idx: torch.Tensor, E: int, BM: int, cap: int):
    import combine_ep_layout_amd as ep
    lib = ep.library()
    T, K = idx.shape
    max_tiles = cap // BM
    d = dev()
    out = {
        "expert_counts": torch.full((E,), -7, dtype=torch.int32, device=d),
        "expert_pool_block_offset": torch.full((E + 1,), -7, dtype=torch.int32, device=d),
        "num_tiles": torch.full((1,), -7, dtype=torch.int32, device=d),
        "tile_expert": torch.full((max_tiles,), -7, dtype=torch.int32, device=d),
        "pool_arrival_target": torch.full((max_tiles,), -7, dtype=torch.int32, device=d),
        "slot_to_pool_row": torch.full((T * K,), -7, dtype=torch.int32, device=d),
        "pool_recv_token": torch.full((cap,), -7, dtype=torch.int32, device=d),
    }
    err = torch.zeros(1, dtype=torch.int32, device=d)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.ep_layout_noalloc(P(idx), T, K, E, BM, cap, P(out["expert_counts"]),
                               P(out["expert_pool_block_offset"]), P(out["num_tiles"]),
                               P(out["tile_expert"]), P(out["pool_arrival_target"]),
                               P(out["slot_to_pool_row"]), P(out["pool_recv_token"]), P(err),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ep.EP_OK, ep.library().ep_status_string(st)
    return out, err


@pytest.mark.parametrize("name,tokens", [("prefill", -1), ("stream", -1), ("share", -1)])
def test_noalloc_layout_equals_layout_twice(name, tokens):
    cfg = CONFIGS[name] if tokens < 0 else CONFIGS[name].replace(tokens=tokens)
    h = new_handle(cfg)
    cap = h.capacity_rows
    # first call at full size, then a smaller batch of another routing
    for call, T in enumerate([cfg.tokens, cfg.tokens // 3 + 5]):
        say(f"[no-alloc] {name}: call {call + 1}, {T} tokens")
        d = generate(cfg.replace(tokens=T), 20 + call)
        idx, w = device_routing(d)
        got, err = _noalloc_layout(idx, cfg.num_experts, cfg.block_m, cap)
        h.layout(idx, w)
        torch.cuda.synchronize()
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m, cap=cap)
        for a in LAYOUT_ARRAYS:
            mine = got[a].cpu().numpy()
            assert np.array_equal(mine, h.array(a).cpu().numpy()), (call, a)
            assert np.array_equal(mine, L[a]), (call, a)
        assert int(got["num_tiles"].cpu()[0]) == L["num_tiles"]
        assert int(err.cpu()[0]) == 0
    h.close()


def test_noalloc_small_then_smaller_and_bad_ids():
    """The one-workgroup path (no scratch) and the multi-workgroup path back
    to back, an out-of-range id reported in the caller's error word, and the
    host-side rejections (nothing is enqueued)."""
    import combine_ep_layout_amd as ep
    lib = ep.library()
    E, BM, K = 64, 16, 4
    cap_t = 9000
    cap = cap_t * K + E * (BM - 1)
    rng = np.random.default_rng(3)
    for call, T in enumerate([cap_t, 300]):
        idx = rng.integers(-1, E, size=(T, K), dtype=np.int32)
        idx[T // 2, 1] = E + 5                       # flagged and treated as masked
        got, err = _noalloc_layout(torch.from_numpy(idx).to(dev()), E, BM, cap)
        torch.cuda.synchronize()
        L = oracle.layout(idx, E, BM, cap=cap)
        for a in LAYOUT_ARRAYS:
            assert np.array_equal(got[a].cpu().numpy(), L[a]), (call, a)
        assert int(err.cpu()[0]) & 1
    P = lambda v: ctypes.c_void_p(v)
    z = torch.zeros(cap, dtype=torch.int32, device=dev())
    zp = z.data_ptr()
    args = [P(zp)] * 7
    INV, UNS = ep.EP_ERR_INVALID_ARGUMENT, ep.EP_ERR_UNSUPPORTED
    # capacity below the worst case, bad sizes, misaligned or missing outputs
    assert lib.ep_layout_noalloc(P(zp), 10, 2, 4, 8, 10, *args, None, None) == INV
    assert lib.ep_layout_noalloc(P(zp), 10, 0, 4, 8, 100, *args, None, None) == INV
    assert lib.ep_layout_noalloc(P(zp), 10, 2, 4, 8, 100, P(zp + 2), *args[1:], None, None) == INV
    assert lib.ep_layout_noalloc(P(zp), 10, 2, 4, 8, 100, None, *args[1:], None, None) == INV
    # a workspace larger than the scratch array: 2^19 tokens x top-32 over 1024 experts
    big_cap = (1 << 19) * 32 + 1024 * 127
    assert lib.ep_layout_noalloc(P(zp), 1 << 19, 32, 1024, 128, big_cap, *args, None, None) == UNS
    torch.cuda.synchronize()
