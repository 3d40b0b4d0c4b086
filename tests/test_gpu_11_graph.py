"""The layout -> dispatch -> combine step captured in a HIP graph (torch's
graph capture on the library's stream) and replayed on new inputs written
into the captured buffers.  Every replay must equal an eager run of the same
inputs bit for bit: the library allocates nothing and sets no memory through
the runtime on the path (all zeroing is done by its own kernels), so a replay
repeats the whole step.  Eager work and synchronisations run between the
replays."""
import numpy as np
import pytest
import torch

from gpu_helpers import say, dev, new_handle, to_dev_bf16, bits_of
from synth import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _eager(cfg, d, eo_bits, fp8):
    h = new_handle(cfg)
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    epoch = h.layout(idx, w)
    pool, scales = h.new_pool(cfg.hidden, fp8=fp8)
    h.dispatch(to_dev_bf16(d["x"]), pool, scales, fp8=fp8)
    y = h.combine(epoch, to_dev_bf16(eo_bits))
    torch.cuda.synchronize()
    out = (pool.view(torch.uint8).cpu().numpy(), None if scales is None else scales.cpu().numpy(),
           bits_of(y), h.array("slot_to_pool_row").cpu().numpy())
    h.close()
    return out


@pytest.mark.parametrize("name,tokens,hidden,fp8", [("tiny", -1, -1, False), ("decode", -1, -1, True),
                                                     ("stream", 3000, 512, False),
                                                     ("share", 4000, 1024, False)])
def test_step_in_graph(name, tokens, hidden, fp8):
    """(3000 stream tokens take the two-launch layout; the share routing is
    sparse, and its combine grid is not resident: before the capture the
    handle's launch-shape hint is set to the density the warm-up layout
    reported, which the test checks against the routing.)"""
    import combine_ep_layout_amd as ep
    say(f"[graph] {name} tokens={tokens} hidden={hidden} fp8={fp8}")
    cfg = CONFIGS[name]
    if tokens >= 0:
        cfg = cfg.replace(tokens=tokens)
    if hidden >= 0:
        cfg = cfg.replace(hidden=hidden)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    cap = h.capacity_rows
    idx = torch.empty(T, K, dtype=torch.int32, device=dev())
    w = torch.empty(T, K, dtype=torch.float32, device=dev())
    x = torch.empty(T, H, dtype=torch.bfloat16, device=dev())
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    pool, scales = h.new_pool(H, fp8=fp8)

    def load(seed):
        d = generate(cfg, seed)
        idx.copy_(torch.from_numpy(d["topk_idx"]))
        w.copy_(torch.from_numpy(d["topk_weights"]))
        x.copy_(to_dev_bf16(d["x"]))
        eo_bits = bits_of(torch.randn(cap, H, generator=torch.Generator().manual_seed(seed))
                          .to(torch.bfloat16))
        eo.copy_(to_dev_bf16(eo_bits))
        return d, eo_bits

    load(0)
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        epoch = h.layout(idx, w)
        h.dispatch(x, pool, scales, fp8=fp8)
        y = h.combine(epoch, eo)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    d0 = generate(cfg, 0)
    dense = (d0["topk_idx"] >= 0).sum() >= 4 * T
    assert h.layout_density() == (ep.EP_DENSITY_DENSE if dense else ep.EP_DENSITY_SPARSE)
    h.set_density_hint(h.layout_density())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        epoch = h.layout(idx, w)
        h.dispatch(x, pool, scales, fp8=fp8)
        h.combine(epoch, eo, y)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        d, eo_bits = load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_pool, want_scales, want_y, want_s2r = _eager(cfg, d, eo_bits, fp8)
        assert np.array_equal(h.array("slot_to_pool_row").cpu().numpy(), want_s2r)
        assert np.array_equal(bits_of(y), want_y)
        real = np.flatnonzero(h.array("pool_recv_token").cpu().numpy() >= 0)
        got_pool = pool.view(torch.uint8).cpu().numpy()
        assert np.array_equal(got_pool[real], want_pool[real])
        if fp8:
            assert np.array_equal(scales.cpu().numpy()[real], want_scales[real])
        say(f"  replay with seed {seed} matches the eager run")
    assert h.sync_status() == 0
    del g
    h.close()


def test_dense_routing_step_in_graph():
    """The dense-routing bf16 dispatch (a read pass over x, then the pool
    stores: two launches) captured with its layout and combine: 8192 tokens x
    hidden 4096 x top-4 (64 MiB of x), the handle's shape hint set to the
    density its warm-up layout reported.  Each replay on new inputs equals an
    eager run of a second handle on the same inputs, compared on the device:
    the row map, y, and every real pool row."""
    import combine_ep_layout_amd as ep
    say("[graph] dense-routing bf16 dispatch, 8192 x 4096 top-4")
    cfg = CONFIGS["prefill"].replace(tokens=8192, hidden=4096, top_k=4)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    ref = new_handle(cfg)
    cap = h.capacity_rows
    idx = torch.empty(T, K, dtype=torch.int32, device=dev())
    w = torch.empty(T, K, dtype=torch.float32, device=dev())
    x = torch.empty(T, H, dtype=torch.bfloat16, device=dev())
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    pool, _ = h.new_pool(H)
    pool_ref, _ = ref.new_pool(H)

    def load(seed):
        d = generate(cfg, seed)
        idx.copy_(torch.from_numpy(d["topk_idx"]))
        w.copy_(torch.from_numpy(d["topk_weights"]))
        x.copy_(to_dev_bf16(d["x"]))
        g = torch.Generator(device=dev())
        g.manual_seed(seed)
        eo.copy_(torch.randn(cap, H, generator=g, device=dev()).to(torch.bfloat16))

    load(0)
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        epoch = h.layout(idx, w)
        h.dispatch(x, pool)
        y = h.combine(epoch, eo)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert h.layout_density() == ep.EP_DENSITY_DENSE
    h.set_density_hint(ep.EP_DENSITY_DENSE)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        epoch = h.layout(idx, w)
        h.dispatch(x, pool)
        h.combine(epoch, eo, y)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        load(seed)
        pool.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e_ref = ref.layout(idx, w)
        ref.dispatch(x, pool_ref)
        y_ref = ref.combine(e_ref, eo)
        torch.cuda.synchronize()
        assert torch.equal(h.array("slot_to_pool_row"), ref.array("slot_to_pool_row"))
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        real = torch.nonzero(ref.array("pool_recv_token") >= 0).flatten()
        assert real.numel() == int((idx >= 0).sum())
        assert torch.equal(pool.view(torch.int16)[real], pool_ref.view(torch.int16)[real])
        say(f"  replay with seed {seed} matches the eager run ({real.numel()} rows)")
    assert h.sync_status() == 0 and ref.sync_status() == 0
    del g
    h.close()
    ref.close()


def test_streaming_dispatch_and_consumer_in_graph():
    """Layout -> streaming FP8 dispatch -> tile consumer captured on one
    stream and replayed on new inputs.  A replay repeats the captured round
    and sequence number: the replayed layout must re-zero the arrival counts
    (else no tile would reach round * target again and the consumer would
    time out) and re-stamp tile_ready below the captured sequence number.
    Every replay's consumer output must equal the dequantised rows of that
    replay's x."""
    import combine_ep_layout_amd as ep
    import oracle
    say("[graph] stream: layout, tile_ready dispatch and consumer, 3 replays")
    cfg = CONFIGS["stream"].replace(tokens=2000, hidden=512)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    h = new_handle(cfg)
    cap = h.capacity_rows
    idx = torch.empty(T, K, dtype=torch.int32, device=dev())
    w = torch.empty(T, K, dtype=torch.float32, device=dev())
    x = torch.empty(T, H, dtype=torch.bfloat16, device=dev())
    pool, scales = h.new_pool(H, fp8=True)
    out = torch.zeros(cap, H, dtype=torch.bfloat16, device=dev())

    def load(seed):
        d = generate(cfg, seed)
        idx.copy_(torch.from_numpy(d["topk_idx"]))
        w.copy_(torch.from_numpy(d["topk_weights"]))
        x.copy_(to_dev_bf16(d["x"]))
        return d

    load(0)
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        h.layout(idx, w)
        seq = h.dispatch(x, pool, scales, fp8=True, tile_ready=True)
        h.tile_consume(seq, pool, scales, H, out, fp8=True, workgroups=16, spin_limit_us=2_000_000)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.layout(idx, w)
        seq = h.dispatch(x, pool, scales, fp8=True, tile_ready=True)
        h.tile_consume(seq, pool, scales, H, out, fp8=True, workgroups=16, spin_limit_us=2_000_000)
    torch.cuda.synchronize()
    for rep in (1, 2, 3):
        d = load(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert h.sync_status() == ep.EP_OK, "a consumer wait timed out"
        L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
        nt = L["num_tiles"]
        ready = h.array("tile_ready").cpu().numpy().view(np.uint32)[:nt]
        cnt = h.array("pool_arrival_count").cpu().numpy().view(np.uint32)[:nt]
        assert (ready == seq).all()
        assert np.array_equal(cnt, L["pool_arrival_target"][:nt].astype(np.uint32))
        real = np.flatnonzero(L["pool_recv_token"] >= 0)
        want = np.stack([oracle.dequant_rows(*[a[None, :] for a in oracle.quantize_row(d["x"][t])])[0]
                         for t in L["pool_recv_token"][real]])
        assert np.array_equal(bits_of(out)[real], want)
        say(f"  replay {rep}: consumer rows match")
    del g
    h.close()


def test_capture_without_layout_is_refused():
    """A streaming dispatch or a gated combine recorded into a graph whose
    capture does not also hold the handle's layout is refused (a replay would
    find the previous replay's arrival and done counts); a plain dispatch is
    accepted, and so is a streaming dispatch captured after its layout."""
    import ctypes
    import combine_ep_layout_amd as ep
    say("[graph] streaming dispatch / gated combine captured without their layout")
    lib = ep.library()
    cfg = CONFIGS["stream"].replace(tokens=600, hidden=512)
    d = generate(cfg, 0)
    H = cfg.hidden
    h = new_handle(cfg)
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    x = to_dev_bf16(d["x"])
    pool, scales = h.new_pool(H, fp8=True)
    eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    y = torch.empty(cfg.tokens, H, dtype=torch.bfloat16, device=dev())
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        epoch = h.layout(idx, w)                         # eager layout
        h.dispatch(x, pool, scales, fp8=True, tile_ready=True)
    torch.cuda.synchronize()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(s.cuda_stream)
    fp8, ready = ep.EP_DISPATCH_FP8, ep.EP_DISPATCH_TILE_READY
    codes = {}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        codes["streaming"] = lib.ep_dispatch(h.raw, P(x), H, P(pool), P(scales), fp8 | ready, sp, None)
        codes["gated"] = lib.ep_combine_gated(h.raw, epoch, P(eo), H, P(y), 1, 1000, sp)
        codes["plain"] = lib.ep_dispatch(h.raw, P(x), H, P(pool), P(scales), fp8, sp, None)
    assert codes["streaming"] == ep.EP_ERR_UNSUPPORTED, codes
    assert codes["gated"] == ep.EP_ERR_UNSUPPORTED, codes
    assert codes["plain"] == ep.EP_OK, codes
    g.replay()
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        h.layout(idx, w)
        h.dispatch(x, pool, scales, fp8=True, tile_ready=True)
    for _ in range(2):
        g2.replay()
        torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    del g, g2
    h.close()


def test_backward_in_graph():
    """combine_grads and dispatch_grads captured in a HIP graph after an eager
    layout (the density hint left at auto, so the capture takes the dense
    shape without waiting) and replayed on new grad_y / expert rows written
    into the captured buffers: every replay equals eager calls on the same
    inputs bit for bit (gradient rows, weight gradients, grad_x)."""
    import combine_ep_layout_amd as ep
    say("[graph] combine_grads + dispatch_grads, 4096 tokens x top-8, hidden 1024")
    cfg = CONFIGS["stream"].replace(tokens=4096, hidden=1024, fp8=False, tile_ready=False)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    d = generate(cfg, 8)
    h = new_handle(cfg)
    cap = h.capacity_rows
    epoch = h.layout(torch.from_numpy(d["topk_idx"]).to(dev()), torch.from_numpy(d["topk_weights"]).to(dev()))
    gy = torch.empty(T, H, dtype=torch.bfloat16, device=dev())
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    geo = torch.zeros(cap, H, dtype=torch.bfloat16, device=dev())
    gw = torch.zeros(T, K, dtype=torch.float32, device=dev())
    gx = torch.zeros(T, H, dtype=torch.bfloat16, device=dev())

    def load(seed):
        gen = torch.Generator(device=dev())
        gen.manual_seed(seed)
        gy.copy_(torch.randn(T, H, generator=gen, device=dev()).to(torch.bfloat16))
        eo.copy_(torch.randn(cap, H, generator=gen, device=dev()).to(torch.bfloat16))

    load(0)
    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm-up outside the capture
        ep.ep_combine_backward(h.raw, epoch, gy, eo, geo, gw)
        ep.ep_dispatch_backward(h.raw, epoch, geo, gx)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ep.ep_combine_backward(h.raw, epoch, gy, eo, geo, gw)
        ep.ep_dispatch_backward(h.raw, epoch, geo, gx)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        geo_e = torch.zeros_like(geo)
        _, gw_e = h.combine_backward(epoch, gy, eo, geo_e)
        gx_e = h.dispatch_backward(epoch, geo_e)
        torch.cuda.synchronize()
        real = torch.from_numpy(np.flatnonzero(h.array("pool_recv_token").cpu().numpy() >= 0)).to(dev())
        assert torch.equal(geo[real].view(torch.int16), geo_e[real].view(torch.int16))
        assert torch.equal(gw.view(torch.int32), gw_e.view(torch.int32))
        assert torch.equal(gx.view(torch.int16), gx_e.view(torch.int16))
        say(f"  replay with seed {seed} matches the eager calls")
    assert h.sync_status() == 0
    del g
    h.close()
