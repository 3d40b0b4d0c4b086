"""Streaming release: per-tile arrival counts and tile_ready stamps acquired by
a consumer on another stream (StreamEP README, "Streaming dispatch in one
paragraph": dispatch release-stores dispatch_seq into tile_ready[tile] once a
tile's pool_arrival_count reaches pool_arrival_target; a consumer on a
different stream acquire-loads tile_ready[tile] >= dispatch_seq and reads the
tile's real rows).

Every consumer wait is bounded (spin_limit_us); a wait that expires shows up
as EP_ERR_TIMEOUT, never as a hang.  Streams may share a hardware queue, which
runs their kernels one after another, so the dispatch is always enqueued
before its consumer: an order that also works serialised.  On separate queues
the consumer starts while the dispatch is still landing rows."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (say, inputs, oracle_layout, new_handle, device_routing, to_dev_bf16,
                         bits_of, dev)

pytestmark = pytest.mark.gpu

SPIN_US = 3_000_000


def _expected_consumer_rows(d, L, fp8, rows):
    recv = L["pool_recv_token"]
    if fp8:
        out = []
        for r in rows:
            q, s = oracle.quantize_row(d["x"][recv[r]])
            out.append(oracle.dequant_rows(q[None, :], s[None, :])[0])
        return np.stack(out)
    return d["x"][recv[rows]]


def _check_end_state(h, L, seq, rounds):
    nt = L["num_tiles"]
    cnt = h.array("pool_arrival_count").cpu().numpy().view(np.uint32)[:nt]
    tgt = L["pool_arrival_target"][:nt].astype(np.uint32)
    assert np.array_equal(cnt, rounds * tgt)
    ready = h.array("tile_ready").cpu().numpy().view(np.uint32)
    assert (ready[:nt] == seq).all()


def _run(name, tokens, fp8, replays=1, sample=None):
    import combine_ep_layout_amd as ep
    cfg, d = inputs(name, tokens)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    h = new_handle(cfg)
    H = cfg.hidden
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()                       # default priority
    h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    pool, scales = h.new_pool(H, fp8=fp8)
    for rep in range(1, replays + 1):
        out = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
        ev = torch.cuda.Event()
        ev.record(sa)                              # layout (and out's zero fill) done
        sb.wait_event(ev)
        seq_next = rep                             # one dispatch per replay, from seq 1
        seq = h.dispatch(x, pool, scales, fp8=fp8, tile_ready=True, stream=sa)
        h.tile_consume(seq_next, pool, scales, H, out, fp8=fp8, workgroups=16,
                       spin_limit_us=SPIN_US, stream=sb)
        assert seq == seq_next
        sb.synchronize()
        sa.synchronize()
        assert h.sync_status() == ep.EP_OK, "a consumer wait timed out"
        _check_end_state(h, L, seq, rep)
        real = np.flatnonzero(L["pool_recv_token"] >= 0)
        if sample is not None:
            real = np.sort(np.random.default_rng(rep).choice(real, size=sample, replace=False))
        got = bits_of(out[torch.from_numpy(real).to(dev())])
        assert np.array_equal(got, _expected_consumer_rows(d, L, fp8, real))
    h.close()


@pytest.mark.parametrize("fp8", [True, False])
def test_consumer_overlapping_small(fp8):
    say(f"[stream] consumer on a second stream, stream tokens=3000 fp8={fp8}")
    _run("stream", 3000, fp8)


def test_replays_without_reset():
    say("[stream] three dispatches on one layout, tile_ready never reset")
    _run("stream", 2500, True, replays=3)


def test_stream_full_size():
    say("[stream] full size, consumer on a second stream, sampled rows")
    _run("stream", -1, True, sample=1024)


def test_bf16_prefill_shape_streaming():
    say("[stream] bf16 prefill shape tokens=1500")
    _run("prefill", 1500, False)


@pytest.mark.parametrize("name,tokens,fp8", [("stream", 2000, True), ("share", 3000, False),
                                              ("decode", -1, True)])
def test_streaming_dispatch_pool_bytes(name, tokens, fp8):
    """With the streaming release on, pool rows and scale bytes are still
    bit-exact and padding rows untouched (device-coherent stores)."""
    from gpu_helpers import full_path_check
    say(f"[stream] pool bytes with tile_ready: {name} tokens={tokens} fp8={fp8}")
    cfg, d = inputs(name, tokens)
    full_path_check(cfg, d, fp8=fp8, tile_ready=True)


def test_layout_stamps_its_tiles_with_the_last_sequence_number():
    """ep_layout sets its tiles' tile_ready to the sequence number of the
    handle's last dispatch, so no tile reads as ready for a dispatch issued
    after the layout.  (A HIP graph replays layout and dispatch with the
    sequence numbers captured, so without this stamp a replayed streaming
    dispatch would find the previous replay's stamps already in place.)"""
    import combine_ep_layout_amd as ep
    say("[stream] layout stamps tile_ready with the last sequence number")
    cfg, d = inputs("stream", 2000)
    _, d2 = inputs("stream", 2000, seed=5)             # a second routing of the same size
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    L2 = oracle.layout(d2["topk_idx"], cfg.num_experts, cfg.block_m)
    h = new_handle(cfg)

    def ready(n):
        return h.array("tile_ready").cpu().numpy().view(np.uint32)[:n]

    h.layout(*device_routing(d))
    assert (ready(L["num_tiles"]) == 0).all()          # no dispatch yet
    pool, scales = h.new_pool(cfg.hidden, fp8=True)
    s1 = h.dispatch(to_dev_bf16(d["x"]), pool, scales, fp8=True, tile_ready=True)
    assert (ready(L["num_tiles"]) == s1).all()
    s2 = h.dispatch(to_dev_bf16(d["x"]), pool, scales, fp8=True)   # not streaming: no stamps
    assert s2 == s1 + 1 and (ready(L["num_tiles"]) == s1).all()
    h.layout(*device_routing(d2))
    assert (ready(L2["num_tiles"]) == s2).all()        # below the next dispatch's number
    s3 = h.dispatch(to_dev_bf16(d2["x"]), pool, scales, fp8=True, tile_ready=True)
    assert s3 == s2 + 1 and (ready(L2["num_tiles"]) == s3).all()
    assert h.sync_status() == ep.EP_OK
    h.close()
