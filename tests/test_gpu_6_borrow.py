"""Borrowed receive view (DeepEP PR #769, Description).  A borrowing
dispatch writes no pool: x itself is the slab and the layout's
pool_recv_token is the row map.  The tests gather rows through that map and
compare them, and the metadata, with the oracle bit for bit; check that the
handle refuses the calls that would disturb a lent view until it is handed
back, and refuses modes a borrow cannot serve before enqueueing anything;
reuse the handle once the view is returned; and keep a reader on another
stream, held back behind other work, reading the old map while a new layout
waits for it."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, generate
from gpu_helpers import (say, inputs, new_handle, device_routing, to_dev_bf16, bits_of,
                         compare_layout, dev, POISON_BF16)

pytestmark = pytest.mark.gpu


def _poisoned_out(h, H):
    return torch.full((h.capacity_rows, H), POISON_BF16 - 0x10000, dtype=torch.int16,
                      device=dev()).view(torch.bfloat16)


@pytest.mark.parametrize("name,tokens", [("share", -1), ("prefill", 1000), ("tiny", -1)])
def test_gathered_view_matches_copied_pool(name, tokens):
    import combine_ep_layout_amd as ep
    say(f"[borrow] gathered view {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    H = cfg.hidden
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    compare_layout(h, L)
    x = to_dev_bf16(d["x"])
    h.borrow(x)
    out = _poisoned_out(h, H)
    h.tile_consume(0, x, None, H, out, gather=True)
    h.release()
    want = oracle.dispatch_bf16(d["x"], L["pool_recv_token"],
                                pool_init=np.full((h.capacity_rows, H), POISON_BF16, np.uint16))
    assert np.array_equal(bits_of(out), want)          # real rows gathered, padding untouched
    # the copying dispatch and its consumer give the same rows
    pool, _ = h.new_pool(H)
    h.dispatch(x, pool)
    out2 = _poisoned_out(h, H)
    h.tile_consume(0, pool, None, H, out2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_lease_rejects_and_release():
    import combine_ep_layout_amd as ep
    say("[borrow] lease rules")
    lib = ep.library()
    cfg, d = inputs("share", 512)
    H = cfg.hidden
    h = new_handle(cfg)
    raw = h.raw
    P = lambda t: None if t is None else t.data_ptr()
    x = to_dev_bf16(d["x"])
    idx, w = device_routing(d)
    pool, _ = h.new_pool(H)
    fpool, fscales = h.new_pool(H, fp8=True)
    y = torch.empty(512, H, dtype=torch.bfloat16, device=dev())
    # no layout yet: nothing to lend
    assert lib.ep_dispatch(raw, P(x), H, None, None, ep.EP_DISPATCH_BORROW, None, None) == ep.EP_ERR_HANDLE_STATE
    epoch = h.layout(idx, w)
    # unsupported modes and bad arguments, rejected before the lease is taken
    assert lib.ep_dispatch(raw, P(x), H, None, None, ep.EP_DISPATCH_BORROW | ep.EP_DISPATCH_FP8,
                           None, None) == ep.EP_ERR_UNSUPPORTED
    assert lib.ep_dispatch(raw, P(x), H, None, None, ep.EP_DISPATCH_BORROW | ep.EP_DISPATCH_TILE_READY,
                           None, None) == ep.EP_ERR_UNSUPPORTED
    assert lib.ep_dispatch(raw, P(x), H, P(pool), None, ep.EP_DISPATCH_BORROW, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(raw, P(x) + 2, H, None, None, ep.EP_DISPATCH_BORROW, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_borrow_release(raw, None) == ep.EP_ERR_HANDLE_STATE
    seq = h.borrow(x)
    assert seq >= 1
    # while the view is out, everything that could disturb it is rejected
    assert lib.ep_dispatch(raw, P(x), H, None, None, ep.EP_DISPATCH_BORROW, None, None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_dispatch(raw, P(x), H, P(pool), None, 0, None, None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_layout(raw, P(idx), P(w), 512, None, None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_combine(raw, epoch, P(pool), H, P(y), None) == ep.EP_ERR_HANDLE_STATE
    assert lib.ep_handle_destroy(raw) == ep.EP_ERR_HANDLE_STATE
    # the consumer may read the view meanwhile
    out = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    h.tile_consume(0, x, None, H, out, gather=True)
    h.release()
    assert lib.ep_borrow_release(raw, None) == ep.EP_ERR_HANDLE_STATE
    # after release: combine, replay of the borrow, a copying dispatch, a new layout
    h.combine(epoch, pool, y)
    h.borrow(x)
    h.release()
    h.dispatch(x, pool)
    assert h.layout(idx, w) == epoch + 1
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_delayed_cross_stream_reader():
    """A consumer delayed behind other work on its own stream still reads the
    row map of the layout it borrowed: the next layout, enqueued at once on the
    handle's stream after release, waits for it."""
    import combine_ep_layout_amd as ep
    say("[borrow] delayed cross-stream reader")
    cfg = CONFIGS["share"]
    d1 = generate(cfg, 0)
    d2 = generate(cfg, 1)
    L1 = oracle.layout(d1["topk_idx"], cfg.num_experts, cfg.block_m)
    H = cfg.hidden
    h = new_handle(cfg)
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()                                   # default priority
    h.layout(*device_routing(d1))
    x = to_dev_bf16(d1["x"])
    h.borrow(x)
    ev = torch.cuda.Event()
    ev.record(sa)
    out = _poisoned_out(h, H)
    busy_a = torch.randn(4096, 4096, device=dev())
    torch.cuda.synchronize()
    with torch.cuda.stream(sb):
        sb.wait_event(ev)
        for _ in range(8):                                     # delay the reader
            busy_a = busy_a @ busy_a
            busy_a = busy_a / busy_a.abs().max()
        h.tile_consume(0, x, None, H, out, gather=True, stream=sb)
    h.release(sb)
    idx2, w2 = device_routing(d2)
    h.layout(idx2, w2)                                          # overwrites the row map after sb
    torch.cuda.synchronize()
    want = oracle.dispatch_bf16(d1["x"], L1["pool_recv_token"],
                                pool_init=np.full((h.capacity_rows, H), POISON_BF16, np.uint16))
    assert np.array_equal(bits_of(out), want)
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_borrow_zero_tokens():
    import combine_ep_layout_amd as ep
    say("[borrow] T=0")
    cfg = CONFIGS["tiny"].replace(tokens=0)
    d = generate(cfg, 0)
    h = new_handle(cfg, max_tokens=16)
    h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    h.borrow(x)
    h.release()
    assert h.sync_status() == ep.EP_OK
    h.close()
