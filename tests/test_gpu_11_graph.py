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
                                                     ("stream", 3000, 512, False)])
def test_step_in_graph(name, tokens, hidden, fp8):
    """(3000 stream tokens take the two-launch layout.)"""
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
