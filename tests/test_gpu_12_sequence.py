"""A long sequence of calls on one handle, each compared with the oracle:
token counts from 0 to the capacity, several hidden sizes, bf16 and FP8,
plain and streaming dispatches (with the per-tile arrival counts checked
against round * target after each one), and routings with masked slots,
repeated experts and tokens with no valid slot.  Nothing of one call may leak
into the next: the epoch, the streaming round, the arrival counts and the
padding rows are all per layout."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (say, dev, to_dev_bf16, bits_of, ulp_diff, compare_layout,
                         POISON_BF16, POISON_U8)
from synth import bf16_from_f32

pytestmark = pytest.mark.gpu


def test_call_sequence_on_one_handle():
    import combine_ep_layout_amd as ep
    rng = np.random.default_rng(11)
    max_t, K, E, BM = 3000, 6, 40, 32
    h = ep.EpHandle(max_t, K, E, BM)
    cap = h.capacity_rows
    last_epoch = 0
    for it in range(24):
        T = [max_t, 0, 1][it] if it < 3 else int(rng.integers(0, max_t + 1))
        H = int(rng.choice([128, 256, 640, 3072]))
        fp8 = bool(rng.integers(0, 2)) and H % 128 == 0
        streaming = bool(rng.integers(0, 2))
        say(f"[sequence] call {it}: T={T} H={H} fp8={fp8} tile_ready={streaming}")
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
        idx[: T // 10] = -1                              # tokens with no valid slot
        w = rng.random((T, K)).astype(np.float32)
        x_bits = bf16_from_f32(rng.standard_normal((T, H), dtype=np.float32))
        L = oracle.layout(idx, E, BM, cap=cap)
        epoch = h.layout(torch.from_numpy(idx).to(dev()), torch.from_numpy(w).to(dev()))
        assert epoch == last_epoch + 1
        last_epoch = epoch
        compare_layout(h, L)
        recv = L["pool_recv_token"]
        real = recv >= 0
        x = to_dev_bf16(x_bits)
        nt = L["num_tiles"]
        # one or two dispatches on this layout; the r-th streaming one brings
        # every tile's arrival count to r * target
        rounds = 0
        for _ in range(int(rng.integers(1, 3))):
            if fp8:
                pool = torch.full((cap, H), POISON_U8, dtype=torch.uint8, device=dev())
                scales = torch.full((cap, H // 128), POISON_U8, dtype=torch.uint8, device=dev())
                h.dispatch(x, pool, scales, fp8=True, tile_ready=streaming)
                op, osc = oracle.dispatch_fp8(x_bits, recv,
                                              pool_init=np.full((cap, H), POISON_U8, np.uint8),
                                              scales_init=np.full((cap, H // 128), POISON_U8,
                                                                  np.uint8))
                assert np.array_equal(pool.cpu().numpy(), op)
                assert np.array_equal(scales.cpu().numpy(), osc)
            else:
                pool = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16,
                                  device=dev()).view(torch.bfloat16)
                h.dispatch(x, pool, None, tile_ready=streaming)
                op = oracle.dispatch_bf16(x_bits, recv,
                                          pool_init=np.full((cap, H), POISON_BF16, np.uint16))
                assert np.array_equal(bits_of(pool), op)
            if streaming:
                rounds += 1
            cnt = h.array("pool_arrival_count").cpu().numpy().view(np.uint32)[:nt]
            tgt = L["pool_arrival_target"][:nt].astype(np.uint32)
            assert np.array_equal(cnt, rounds * tgt)
        # combine on seeded expert rows; rows no slot owns hold NaN
        eo_bits = bf16_from_f32(rng.standard_normal((cap, H), dtype=np.float32))
        eo_bits[~real] = 0x7FC0
        y = h.combine(epoch, to_dev_bf16(eo_bits))
        y_or = oracle.combine(eo_bits, L["slot_to_pool_row"], w)
        got = bits_of(y)
        assert got.shape == y_or.shape
        assert ulp_diff(got, y_or).max(initial=0) <= 1
        assert h.sync_status() == (ep.EP_ERR_BAD_ROUTING if L["error"] else ep.EP_OK)
    h.close()
