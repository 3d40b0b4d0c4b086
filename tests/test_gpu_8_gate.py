"""Per-token combine gate (StreamEP README, opening paragraph: combine is
gated per receive token by y_done_per_token, so it can start on a token as
soon as that token's expert compute has drained).

The expert-output producer is the tile consumer stand-in with
EP_CONSUME_SIGNAL_DONE: it copies (or dequantises) each tile's rows into
expert_out, publishes them at device scope and adds 1 to the done count of
each row's token.  ep_combine_gated waits per token for round * (unmasked
slots) and must then equal the ungated combine bit for bit.  Every wait is
bounded; an expired wait shows up as EP_ERR_TIMEOUT, never as a hang."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (say, inputs, new_handle, device_routing, to_dev_bf16, bits_of, dev,
                         POISON_BF16)

pytestmark = pytest.mark.gpu

SPIN_US = 3_000_000


def _slots_per_token(L, T, K):
    return (L["slot_to_pool_row"].reshape(T, K) >= 0).sum(1).astype(np.uint32)


def _expected_y(d, L, fp8):
    """Oracle combine of the producer's rows: copies of x (bf16) or the
    dequantised FP8 rows; padding rows are NaN and never read."""
    from oracle import par as oracle_par
    recv = L["pool_recv_token"]
    H = d["x"].shape[1]
    eo = np.full((recv.size, H), 0x7FC0, np.uint16)
    real = np.flatnonzero(recv >= 0)
    if fp8:
        q_tok, s_tok = oracle_par.quantize_tokens(d["x"])
        eo[real] = oracle_par.dequant_tokens(q_tok, s_tok)[recv[real]]
    else:
        eo[real] = d["x"][recv[real]]
    return oracle_par.combine(eo, L["slot_to_pool_row"], d["topk_weights"])


def _pipeline(name, tokens, fp8, rounds=1, one_stream=False, top_k=None):
    """layout on A; then per round: dispatch (tile_ready) on A, the producer on
    B and the gated combine on C, enqueued in that order.  Streams may share a
    hardware queue, which runs their kernels one after another, so the
    enqueue order is always one that also works serialised.  The producer
    waits only for the layout and overlaps the dispatch; the combine starts
    once the dispatch has ended (no dispatch workgroup has to find room beside
    spinning combine waves) and waits on tokens the producer is still
    writing.  With one_stream everything runs in order on A."""
    import combine_ep_layout_amd as ep
    cfg, d = inputs(name, tokens)
    if top_k is not None:                       # the same tokens, routed to top_k experts
        from synth import generate
        cfg = cfg.replace(top_k=top_k)
        d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    want = _expected_y(d, L, fp8)
    h = new_handle(cfg)
    sa = torch.cuda.current_stream()
    sb, sc = (sa, sa) if one_stream else (torch.cuda.Stream(), torch.cuda.Stream())  # default priority
    epoch = h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    pool, scales = h.new_pool(H, fp8=fp8)
    for rnd in range(1, rounds + 1):
        eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
        y = torch.full((T, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
        ev = torch.cuda.Event()
        ev.record(sa)                       # layout, eo's and y's fills are done
        sb.wait_event(ev)
        h.dispatch(x, pool, scales, fp8=fp8, tile_ready=True, stream=sa)
        h.tile_consume(rnd, pool, scales, H, eo, fp8=fp8, workgroups=16,
                       spin_limit_us=SPIN_US, stream=sb, signal_done=True)
        if not one_stream:
            ev_d = torch.cuda.Event()
            ev_d.record(sa)
            sc.wait_event(ev_d)
        h.combine_gated(epoch, eo, round=rnd, y=y, spin_limit_us=SPIN_US, stream=sc)
        for s in (sa, sb, sc):
            s.synchronize()
        assert h.sync_status() == ep.EP_OK, "a bounded wait timed out"
        done = h.array("y_done_per_token").cpu().numpy().view(np.uint32)
        assert np.array_equal(done, rnd * _slots_per_token(L, T, K))
        assert np.array_equal(bits_of(y), want)
        # the ungated combine of the same rows agrees bit for bit
        assert np.array_equal(bits_of(h.combine(epoch, eo)), want)
    h.close()


@pytest.mark.parametrize("name,tokens,fp8", [("tiny", -1, False), ("decode", -1, True),
                                              ("share", 3000, False), ("prefill", 1000, False)])
def test_gate_after_producer(name, tokens, fp8):
    say(f"[gate] producer finishes first: {name} tokens={tokens} fp8={fp8}")
    _pipeline(name, tokens, fp8, one_stream=True)


@pytest.mark.parametrize("name,tokens,fp8", [("decode", -1, True), ("share", 3000, False),
                                              ("stream", 2000, True)])
def test_gate_concurrent_streams(name, tokens, fp8):
    """Producer and gated combine run at the same time on two streams, next to
    the dispatch on a third; the combine waits on tokens whose rows are still
    being written."""
    say(f"[gate] concurrent: {name} tokens={tokens} fp8={fp8}")
    _pipeline(name, tokens, fp8)


@pytest.mark.parametrize("name,fp8", [("prefill", False), ("stream", True)])
def test_gate_full_size(name, fp8):
    """The prefill and streaming workloads at full size, in order on one
    stream: dense batches hold several items' stores, and every wave owns
    several items.  Every element of y against the oracle."""
    say(f"[gate] full size {name}, in order")
    _pipeline(name, -1, fp8, one_stream=True)


@pytest.mark.parametrize("top_k,one_stream", [(16, True), (32, True), (16, False), (32, False)])
def test_gate_top_k_above_8(top_k, one_stream):
    """top_k 16 and 32: the gated combine walks a token's slots in groups of
    8, in order and with the producer and combine on their own streams."""
    say(f"[gate] top_k={top_k} one_stream={one_stream}")
    _pipeline("stream", 900, False, one_stream=one_stream, top_k=top_k)


def test_gate_rounds_without_relayout():
    say("[gate] three producer rounds on one layout, counts never reset")
    _pipeline("share", 2000, False, rounds=3)


def test_gate_timeout_is_bounded_and_reported():
    """No producer runs: every token with a slot times out (the first expiry
    makes the others give up at once) and keeps its old y row; tokens without
    a slot are written (+0).  The handle works normally afterwards."""
    import combine_ep_layout_amd as ep
    say("[gate] timeout with no producer")
    cfg, d = inputs("share", 3000)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    n_t = _slots_per_token(L, T, K)
    assert (n_t == 0).any() and (n_t > 0).any()
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    y = torch.full((T, H), POISON_BF16 - 0x10000, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    h.combine_gated(epoch, eo, round=1, y=y, spin_limit_us=2000)
    assert h.sync_status() == ep.EP_ERR_TIMEOUT
    got = bits_of(y)
    assert (got[n_t == 0] == 0).all()
    assert (got[n_t > 0] == POISON_BF16).all()
    assert h.sync_status() == ep.EP_OK                       # cleared by the first read
    _pipeline("share", 3000, False)
    h.close()


def test_gate_rejections():
    import combine_ep_layout_amd as ep
    say("[gate] rejections")
    lib = ep.library()
    cfg, d = inputs("tiny")
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    H = cfg.hidden
    eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    y = torch.empty(cfg.tokens, H, dtype=torch.bfloat16, device=dev())
    P = lambda t: t.data_ptr()
    assert lib.ep_combine_gated(h.raw, epoch, P(eo), H, P(y), 0, 1000, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_combine_gated(h.raw, epoch + 1, P(eo), H, P(y), 1, 1000, None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_combine_gated(h.raw, epoch, P(eo) + 8, H, P(y), 1, 1000, None) == ep.EP_ERR_INVALID_ARGUMENT
    h.borrow(to_dev_bf16(d["x"]))
    assert lib.ep_combine_gated(h.raw, epoch, P(eo), H, P(y), 1, 1000, None) == ep.EP_ERR_HANDLE_STATE
    h.release()
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    h.close()


@pytest.mark.parametrize("T,H,K,E,BM", [(1, 128, 1, 1, 1), (37, 256, 3, 5, 1), (64, 512, 2, 1, 7)])
def test_gate_small_shapes(T, H, K, E, BM):
    """One token, one expert, BLOCK_M 1, odd top-k: the gate's batch and
    stride arithmetic at the smallest shapes (some tokens have no slot)."""
    import combine_ep_layout_amd as ep
    from synth import Config, generate
    say(f"[gate] small shape T={T} H={H} K={K} E={E} BM={BM}")
    cfg = Config("gate_edge", T, H, K, E, E, BM)
    d = generate(cfg, 4)
    if E == 1:
        idx = np.zeros((T, K), np.int32)
        idx[::3, -1] = -1
        d["topk_idx"] = idx
    L = oracle.layout(d["topk_idx"], E, BM)
    want = _expected_y(d, L, False)
    h = new_handle(cfg)
    epoch = h.layout(*device_routing(d))
    pool, _ = h.new_pool(H)
    eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    seq = h.dispatch(to_dev_bf16(d["x"]), pool, tile_ready=True)
    h.tile_consume(seq, pool, None, H, eo, workgroups=3, spin_limit_us=SPIN_US, signal_done=True)
    y = h.combine_gated(epoch, eo, round=1, spin_limit_us=SPIN_US)
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    assert np.array_equal(bits_of(y), want)
    done = h.array("y_done_per_token").cpu().numpy().view(np.uint32)
    assert np.array_equal(done, _slots_per_token(L, T, K))
    h.close()


@pytest.mark.parametrize("sync", [True, False])
def test_gate_after_dense_and_sparse_layouts(sync):
    """The gated combine's batch shape follows the routing density the layout
    reports (dense batches hold several items' stores); the results do not
    depend on it.  One handle alternates a dense and a sparse routing of the
    same size, with or without a synchronisation after each layout (without
    it the density in force may still be the previous layout's), and every
    gated combine is compared with the oracle."""
    import combine_ep_layout_amd as ep
    from synth import CONFIGS, generate
    say(f"[gate] alternating dense / sparse layouts on one handle, sync={sync}")
    dense = CONFIGS["stream"].replace(tokens=6000, hidden=1024, mask_frac=0.0, fp8=False,
                                      tile_ready=False)
    sparse = CONFIGS["share"].replace(tokens=6000, hidden=1024, num_experts=128, experts_global=128,
                                      local_keep=16)
    h = new_handle(dense)
    H = dense.hidden
    pool, _ = h.new_pool(H)
    for it, cfg in enumerate([dense, sparse, dense, sparse]):
        d = generate(cfg, 60 + it)
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m, cap=h.capacity_rows)
        want = _expected_y(d, L, False)
        epoch = h.layout(*device_routing(d))
        if sync:
            torch.cuda.synchronize()
        eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
        seq = h.dispatch(to_dev_bf16(d["x"]), pool, tile_ready=True)
        h.tile_consume(seq, pool, None, H, eo, workgroups=64, spin_limit_us=SPIN_US,
                       signal_done=True)
        y = h.combine_gated(epoch, eo, round=1, spin_limit_us=SPIN_US)
        torch.cuda.synchronize()
        assert h.sync_status() == ep.EP_OK
        assert np.array_equal(bits_of(y), want), it
        say(f"  layout {it}: {(d['topk_idx'] >= 0).sum() / cfg.tokens:.2f} rows per token, match")
    h.close()
