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


def _check_end_state(h, L, seq, rounds):
    nt = L["num_tiles"]
    cnt = h.array("pool_arrival_count").cpu().numpy().view(np.uint32)[:nt]
    tgt = L["pool_arrival_target"][:nt].astype(np.uint32)
    assert np.array_equal(cnt, rounds * tgt)
    ready = h.array("tile_ready").cpu().numpy().view(np.uint32)
    assert (ready[:nt] == seq).all()


def _check_rows(d, L, fp8, out, pool, scales, per_token):
    """Every real row: the consumer's output against the oracle (a copy of x,
    or the dequantised codes of its token), and the pool bytes and scales the
    streaming dispatch left behind against the oracle's per-token
    quantisation."""
    recv = L["pool_recv_token"]
    real = np.flatnonzero(recv >= 0)
    step = 32768
    for r0 in range(0, len(real), step):
        rows = real[r0:r0 + step]
        rt = torch.from_numpy(rows).to(dev())
        toks = recv[rows]
        if fp8:
            q_tok, s_tok, deq_tok = per_token
            assert np.array_equal(bits_of(out[rt]), deq_tok[toks]), r0
            assert np.array_equal(pool[rt].cpu().numpy(), q_tok[toks]), r0
            assert np.array_equal(scales[rt].cpu().numpy(), s_tok[toks]), r0
        else:
            assert np.array_equal(bits_of(out[rt]), d["x"][toks]), r0
            assert np.array_equal(bits_of(pool[rt]), d["x"][toks]), r0


def _run(name, tokens, fp8, replays=1, top_k=None):
    import combine_ep_layout_amd as ep
    from oracle import par as oracle_par
    cfg, d = inputs(name, tokens)
    if top_k is not None:                       # the same tokens, routed to top_k experts
        cfg = cfg.replace(top_k=top_k)
        from synth import generate
        d = generate(cfg, 0)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    per_token = None
    if fp8:
        q_tok, s_tok = oracle_par.quantize_tokens(d["x"])
        per_token = (q_tok, s_tok, oracle_par.dequant_tokens(q_tok, s_tok))
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
        _check_rows(d, L, fp8, out, pool, scales, per_token)
    h.close()


@pytest.mark.parametrize("fp8", [True, False])
def test_consumer_overlapping_small(fp8):
    say(f"[stream] consumer on a second stream, stream tokens=3000 fp8={fp8}")
    _run("stream", 3000, fp8)


def test_replays_without_reset():
    say("[stream] three dispatches on one layout, tile_ready never reset")
    _run("stream", 2500, True, replays=3)


def test_stream_full_size():
    say("[stream] full size, consumer on a second stream, every row")
    _run("stream", -1, True)


@pytest.mark.parametrize("top_k,fp8", [(16, True), (32, True), (16, False), (32, False)])
def test_streaming_dispatch_top_k_above_8(top_k, fp8):
    """top_k 16 and 32: the dispatch walks a token's slots in groups of 8;
    every pool row, scale row and consumer row against the oracle."""
    say(f"[stream] top_k={top_k} fp8={fp8}, 700 tokens")
    _run("stream", 700, fp8, top_k=top_k)


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


def _spearman(a, b):
    ra = np.argsort(np.argsort(a)).astype(np.float64)
    rb = np.argsort(np.argsort(b)).astype(np.float64)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / np.sqrt((ra * ra).sum() * (rb * rb).sum()))


def test_consumer_overlaps_dispatch_in_token_order():
    """Full stream workload, consumer (256 workgroups, acquire stamps on) on a
    second stream enqueued right after the streaming dispatch.  Every row is
    checked.  When the consumer's stream started before the dispatch ended
    (they did not share a hardware queue), some tiles must have been seen not
    ready and then ready -- the consumer ran while rows were landing -- and
    those tiles must have become ready in the order the dispatch writes
    tokens: their acquire clocks rank-correlate with the last token each tile
    holds."""
    import combine_ep_layout_amd as ep
    from oracle import par as oracle_par
    say("[stream] consumer overlapping the dispatch, acquire stamps")
    cfg, d = inputs("stream")
    L = oracle_layout("stream")
    q_tok, s_tok = oracle_par.quantize_tokens(d["x"])
    per_token = (q_tok, s_tok, oracle_par.dequant_tokens(q_tok, s_tok))
    h = new_handle(cfg)
    H = cfg.hidden
    sa, sb = torch.cuda.current_stream(), torch.cuda.Stream()      # default priority
    h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    pool, scales = h.new_pool(H, fp8=True)
    out = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    ev = torch.cuda.Event()
    ev.record(sa)
    sb.wait_event(ev)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(sa)
    seq = h.dispatch(x, pool, scales, fp8=True, tile_ready=True, stream=sa)
    d1.record(sa)
    c0.record(sb)
    h.tile_consume(seq, pool, scales, H, out, fp8=True, workgroups=256, spin_limit_us=SPIN_US,
                   stream=sb, stamps=True)
    c1.record(sb)
    sa.synchronize()
    sb.synchronize()
    assert h.sync_status() == ep.EP_OK, "a consumer wait timed out"
    _check_end_state(h, L, seq, 1)
    _check_rows(d, L, True, out, pool, scales, per_token)
    nt = L["num_tiles"]
    st = h.array("tile_stamp").cpu().numpy().view(np.uint64)[:nt]
    waited = (st >> np.uint64(63)).astype(bool)
    clock = (st & np.uint64((1 << 63) - 1)).astype(np.int64)
    started_before_end = c0.elapsed_time(d1) > 0          # consumer stream began before the dispatch ended
    say(f"  dispatch {d0.elapsed_time(d1) * 1e3:.1f} us; consumer began "
        f"{d0.elapsed_time(c0) * 1e3:.1f} us after the dispatch, ended "
        f"{d0.elapsed_time(c1) * 1e3:.1f} us after it; tiles seen not ready first: "
        f"{int(waited.sum())} of {nt}")
    if not started_before_end:
        say("  the two streams ran one after the other (shared hardware queue): no overlap to check")
        h.close()
        return
    assert waited.sum() >= 16
    recv = L["pool_recv_token"]
    last_tok = np.array([recv[j * cfg.block_m:(j + 1) * cfg.block_m].max() for j in range(nt)])
    rho = _spearman(clock[waited], last_tok[waited])
    say(f"  rank correlation of acquire clock and last token, waited tiles: {rho:.3f}")
    assert rho > 0.8
    h.close()
