"""FP8 variants (instagit DeepEP low-latency page: use_ue8m0, round_scale and
per_token_cast_back): float32 and power-of-two float32 scales, the MN-major
scale layout (UE8M0 packed four groups to a word), and the GPU cast back.
Codes and scales are compared with the oracle byte for byte, padding rows and
unused scale columns must stay untouched, and the cast back is bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from synth import bf16_from_f32
from gpu_helpers import (say, inputs, new_handle, device_routing, to_dev_bf16, bits_of, dev,
                         POISON_U8)

pytestmark = pytest.mark.gpu

KINDS = ["ue8m0", "f32", "pow2_f32"]
POISON_F32 = np.float32(-3.25)          # never a scale the dispatch writes (scales are >= 0)
POISON_WORD = 0xA5A5A5A5


def _poison_scales(h, H, kind, mn):
    import combine_ep_layout_amd as ep
    shape, dtype = h.scale_shape(H, kind, mn)
    if dtype == torch.uint8:
        host = np.full(shape, POISON_U8, np.uint8)
    elif dtype == torch.int32:
        host = np.full(shape, POISON_WORD, np.uint32)
    else:
        host = np.full(shape, POISON_F32, np.float32)
    t = torch.from_numpy(host.view(np.int32) if dtype == torch.int32 else host).to(dev())
    return t, host


def _scales_host(t, host_like):
    a = t.cpu().numpy()
    return a.view(np.uint32) if host_like.dtype == np.uint32 else a


def _dispatch_check(cfg, d, kind, mn, tile_ready=False, per_token=None):
    """Dispatch on the GPU and compare pool bytes and scales with the oracle.
    Returns the handle, pool, scales and the oracle layout for further use."""
    H = cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    cap = h.capacity_rows
    recv = L["pool_recv_token"]
    pool = torch.full((cap, H), POISON_U8, dtype=torch.uint8, device=dev())
    scales, s_init = _poison_scales(h, H, kind, mn)
    h.dispatch(to_dev_bf16(d["x"]), pool, scales, fp8=True, tile_ready=tile_ready,
               scale_kind=kind, mn_major=mn)
    got_p = pool.cpu().numpy()
    got_s = _scales_host(scales, s_init)
    if per_token is None:
        op, osc = oracle.dispatch_fp8_scaled(d["x"], recv, kind, mn, ld=h.scale_ld,
                                             pool_init=np.full((cap, H), POISON_U8, np.uint8),
                                             scales_init=s_init)
        assert np.array_equal(got_p, op)
        if got_s.dtype == np.float32:
            assert np.array_equal(got_s.view(np.uint32), osc.view(np.uint32))
        else:
            assert np.array_equal(got_s, osc)
    else:
        # full size: every real row against the oracle's quantisation of its
        # token (computed once per token), every padding row untouched
        from oracle import par as oracle_par
        real = np.flatnonzero(recv >= 0)
        q_tok, s_tok = per_token
        G = H // 128
        step = 16384
        for r0 in range(0, real.size, step):
            rows = real[r0:r0 + step]
            toks = recv[rows]
            assert np.array_equal(got_p[rows], q_tok[toks]), r0
            if mn and kind == "ue8m0":
                # the rows' columns of the packed words, read back as little-endian bytes
                cols = np.ascontiguousarray(got_s[:, rows].T).astype("<u4")
                rm = cols.view(np.uint8).reshape(rows.size, -1)[:, :G]
            elif mn:
                rm = got_s[:, rows].T
            else:
                rm = got_s[rows]
            if kind == "ue8m0":
                assert np.array_equal(rm, s_tok[toks]), r0
            else:
                assert np.array_equal(np.ascontiguousarray(rm).view(np.uint32),
                                      s_tok[toks].view(np.uint32)), r0
        pad = np.flatnonzero(recv < 0)
        assert (got_p[pad] == POISON_U8).all()
        if mn:
            unused = np.ones(got_s.shape[1], bool)
            unused[real] = False
            assert np.array_equal(got_s[:, unused], s_init[:, unused])
        else:
            assert np.array_equal(got_s[pad], s_init[pad])
    return h, pool, scales, L


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mn", [False, True])
@pytest.mark.parametrize("name,tokens", [("tiny", -1), ("decode", -1), ("share", 2000),
                                         ("prefill", 600)])
def test_scaled_dispatch_parity(kind, mn, name, tokens):
    say(f"[fp8var] dispatch {name} tokens={tokens} kind={kind} mn={mn}")
    cfg, d = inputs(name, tokens)
    h, pool, scales, L = _dispatch_check(cfg, d, kind, mn)
    # cast back every row (padding rows hold poison codes and scales: any input is defined)
    cap, H = h.capacity_rows, cfg.hidden
    out = torch.empty(cap, H, dtype=torch.bfloat16, device=dev())
    import combine_ep_layout_amd as ep
    ep.cast_back(pool, scales, kind, mn, rows=cap, out=out)
    s_host = _scales_host(scales, np.zeros(1, np.uint32 if (mn and kind == "ue8m0") else np.uint8))
    want = oracle.cast_back(pool.cpu().numpy(), s_host, kind, mn)
    assert np.array_equal(bits_of(out), want)
    h.close()


@pytest.mark.parametrize("kind", KINDS)
def test_scaled_dispatch_streaming_release(kind):
    """The device-coherent stores of the streaming release write the same
    bytes, and tiles still reach their targets."""
    say(f"[fp8var] streaming dispatch kind={kind} MN-major")
    cfg, d = inputs("stream", 2000)
    h, _, _, L = _dispatch_check(cfg, d, kind, True, tile_ready=True)
    nt = L["num_tiles"]
    cnt = h.array("pool_arrival_count").cpu().numpy().view(np.uint32)[:nt]
    assert np.array_equal(cnt, L["pool_arrival_target"][:nt].astype(np.uint32))
    assert (h.array("tile_ready").cpu().numpy()[:nt] == 1).all()
    h.close()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mn", [False, True])
def test_streaming_consumer_every_flavour(kind, mn):
    """Streaming dispatch in each flavour and layout with the tile consumer on a
    second stream: every real row it writes equals the oracle's cast back of
    the oracle's quantised row."""
    import combine_ep_layout_amd as ep
    say(f"[fp8var] streaming consumer kind={kind} mn={mn}")
    cfg, d = inputs("stream", 2000)
    H = cfg.hidden
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    recv = L["pool_recv_token"]
    real = np.flatnonzero(recv >= 0)
    h = new_handle(cfg)
    sa, sb = torch.cuda.current_stream(), torch.cuda.Stream()          # default priority
    h.layout(*device_routing(d))
    pool, scales = h.new_pool(H, fp8=True, scale_kind=kind, mn_major=mn)
    out = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    ev = torch.cuda.Event()
    ev.record(sa)
    sb.wait_event(ev)
    seq = h.dispatch(to_dev_bf16(d["x"]), pool, scales, fp8=True, tile_ready=True,
                     scale_kind=kind, mn_major=mn, stream=sa)
    h.tile_consume(seq, pool, scales, H, out, fp8=True, workgroups=16, spin_limit_us=3_000_000,
                   stream=sb, scale_kind=kind, mn_major=mn)
    sa.synchronize()
    sb.synchronize()
    assert h.sync_status() == ep.EP_OK
    op, osc = oracle.dispatch_fp8_scaled(d["x"][recv[real]], np.arange(real.size, dtype=np.int32), kind)
    want = oracle.cast_back(op, osc, kind)
    got = bits_of(out[torch.from_numpy(real).to(dev())])
    assert np.array_equal(got, want)
    h.close()


@pytest.mark.parametrize("kind", KINDS)
def test_scaled_dispatch_full_size(kind):
    """The prefill workload at full size in each flavour and both scale
    layouts: every pool row and scale against the oracle."""
    from oracle import par as oracle_par
    cfg, d = inputs("prefill")
    per_token = oracle_par.quantize_tokens(d["x"], kind=kind)
    for mn in (False, True):
        say(f"[fp8var] prefill full size kind={kind} mn={mn}, every row")
        h, pool, scales, L = _dispatch_check(cfg, d, kind, mn, per_token=per_token)
        del pool, scales
        h.close()


def test_special_values_all_flavours():
    """Zero, subnormal-amax, huge, infinite and NaN groups through every
    flavour and layout, and the cast back of every code."""
    from synth import Config, generate
    say("[fp8var] special values")
    rng = np.random.default_rng(21)
    T, H = 24, 1024
    cfg = Config("special", T, H, 2, 4, 4, 16)
    d = generate(cfg, 3)
    x32 = (rng.standard_normal((T, H)) * 2.0 ** rng.integers(-30, 30, (T, 1))).astype(np.float32)
    x32[0] = 0.0
    x32[1, :128] = -0.0
    x32[2] *= np.float32(2.0 ** -120)
    x32[3, :256] = np.float32(3e38)
    x32[4, 5] = np.inf
    x32[5, 700] = -np.inf
    x32[6, 9] = np.nan
    x32[7, :128] = np.nan
    x32[8] *= np.float32(2.0 ** -133)
    d["x"] = bf16_from_f32(x32)
    d["x"][9, 3] = 0x0001                    # smallest bf16 subnormal
    for kind in KINDS:
        for mn in (False, True):
            h, pool, scales, L = _dispatch_check(cfg, d, kind, mn)
            h.close()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mn", [False, True])
def test_cast_back_every_code(kind, mn):
    """Every code 0..255 in every group, against scales spanning the range
    (subnormal and overflowing products, zero and infinite float scales)."""
    import combine_ep_layout_amd as ep
    say(f"[fp8var] cast back every code kind={kind} mn={mn}")
    rows, H = 40, 256
    G = H // 128
    q = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    rng = np.random.default_rng(22)
    if kind == "ue8m0":
        rm = rng.integers(0, 256, size=(rows, G), dtype=np.uint8)
        rm[0] = 0
        rm[1] = 254
        rm[2] = 255
    elif kind == "pow2_f32":
        rm = oracle.pow2_scales_from_ue8m0(rng.integers(0, 255, size=(rows, G)).astype(np.uint8))
    else:
        rm = (rng.standard_normal((rows, G)) * 2.0 ** rng.integers(-140, 120, (rows, G))).astype(np.float32)
        rm = np.abs(rm)
        rm[0] = 0.0
        rm[1] = np.inf
        rm[2] = np.float32(2.0 ** -149)
        rm[3] = np.float32(3.4e38)
    ld = rows + 4
    s_host = oracle.scales_to_mn_major(rm, ld) if mn else rm
    s_dev = torch.from_numpy(s_host.view(np.int32) if s_host.dtype == np.uint32 else s_host).to(dev())
    q_dev = torch.from_numpy(q).to(dev())
    out = ep.cast_back(q_dev, s_dev, kind, mn, rows=rows)
    want = oracle.cast_back(q, s_host, kind, mn)
    assert np.array_equal(bits_of(out), want)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mn", [False, True])
def test_cast_back_ragged_unit_groups(kind, mn):
    """The cast back stores each group of 64 decoded 16-channel units as two
    1 KB runs; a row's last group may hold fewer units (hidden 640: 40,
    896: 56, 1152: 8, 1920: 56) or exactly fill it (hidden 65536, the
    largest), so only part of the runs is stored.  Every code value, random
    scales, rows against the oracle bit for bit."""
    import combine_ep_layout_amd as ep
    rng = np.random.default_rng(31)
    for H, rows in ((640, 37), (896, 29), (1152, 33), (1920, 21), (65536, 3)):
        say(f"[fp8var] cast back ragged groups kind={kind} mn={mn} hidden={H} rows={rows}")
        G = H // 128
        q = rng.integers(0, 256, size=(rows, H), dtype=np.uint8)
        if kind == "ue8m0":
            rm = rng.integers(100, 160, size=(rows, G), dtype=np.uint8)
        elif kind == "pow2_f32":
            rm = oracle.pow2_scales_from_ue8m0(rng.integers(100, 160, size=(rows, G)).astype(np.uint8))
        else:
            rm = np.abs(rng.standard_normal((rows, G))).astype(np.float32) + np.float32(0.01)
        s_host = oracle.scales_to_mn_major(rm, rows + 3) if mn else rm
        s_dev = torch.from_numpy(s_host.view(np.int32) if s_host.dtype == np.uint32 else s_host).to(dev())
        out = ep.cast_back(torch.from_numpy(q).to(dev()), s_dev, kind, mn, rows=rows)
        assert np.array_equal(bits_of(out), oracle.cast_back(q, s_host, kind, mn)), H


def test_fp8_variant_rejections():
    import combine_ep_layout_amd as ep
    say("[fp8var] rejections")
    lib = ep.library()
    cfg, d = inputs("tiny")
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    H = cfg.hidden
    x = to_dev_bf16(d["x"])
    pool = torch.empty(h.capacity_rows, H, dtype=torch.uint8, device=dev())
    sc = torch.empty(h.capacity_rows * (H // 128) + 4, dtype=torch.float32, device=dev())
    P = lambda t: t.data_ptr()
    F8 = ep.EP_DISPATCH_FP8
    # scale flags without FP8, misaligned float scales
    assert lib.ep_dispatch(h.raw, P(x), H, P(pool), None, ep.EP_SCALE_F32, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(h.raw, P(x), H, P(pool), P(sc) + 2, F8 | ep.EP_SCALE_F32, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(h.raw, P(x), H, P(pool), P(sc) + 2, F8 | ep.EP_SCALE_MN_MAJOR, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    # the tile consumer: scale flags need FP8 and aligned float scales
    out = torch.empty(h.capacity_rows, H, dtype=torch.bfloat16, device=dev())
    assert lib.ep_tile_consume(h.raw, 1, P(pool), P(sc), H, ep.EP_SCALE_F32, P(out), 4, 1000,
                               None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_tile_consume(h.raw, 1, P(pool), P(sc) + 2, H, F8 | ep.EP_SCALE_F32, P(out), 4, 1000,
                               None) == ep.EP_ERR_INVALID_ARGUMENT
    # cast back: hidden not a multiple of 128, leading dimension below rows, unknown flag
    q = torch.zeros(8, 256, dtype=torch.uint8, device=dev())
    o = torch.empty(8, 256, dtype=torch.bfloat16, device=dev())
    s8 = torch.zeros(8, 2, dtype=torch.uint8, device=dev())
    assert lib.ep_fp8_cast_back(P(q), P(s8), 0, 8, 0, 192, P(o), None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_fp8_cast_back(P(q), P(s8), ep.EP_SCALE_MN_MAJOR, 8, 7, 256, P(o), None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_fp8_cast_back(P(q), P(s8), ep.EP_DISPATCH_TILE_READY, 8, 0, 256, P(o), None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_fp8_cast_back(None, None, 0, 0, 0, 256, None, None) == ep.EP_OK      # zero rows
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK
    h.close()


@pytest.mark.parametrize("kind", ["ue8m0", "pow2_f32"])
def test_cast_back_every_code_every_scale(kind):
    """Every code against every power-of-two scale (UE8M0 bytes 0..255; float
    2^e for e = -127..127), the range where the hardware conversion decodes:
    bit-identical to the oracle, NaN codes keeping their sign."""
    import combine_ep_layout_amd as ep
    say(f"[fp8var] cast back: every code x every scale, {kind}")
    H = 256
    nb = 256 if kind == "ue8m0" else 255
    q = np.tile(np.arange(256, dtype=np.uint8), (nb, 1))            # row b: codes 0..255
    b = np.arange(nb, dtype=np.uint8)
    rm = np.stack([b, b], axis=1)                                     # both groups of row b
    if kind == "pow2_f32":
        rm = oracle.pow2_scales_from_ue8m0(rm)
    out = ep.cast_back(torch.from_numpy(q).to(dev()), torch.from_numpy(np.ascontiguousarray(rm)).to(dev()),
                       kind, False)
    assert np.array_equal(bits_of(out), oracle.cast_back(q, rm, kind))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mn", [False, True])
def test_fp8_variants_one_group_rows(kind, mn):
    """hidden 128 (one group, a packed word with three zero bytes), top-1,
    BLOCK_M 1, one-unit items: dispatch, streaming dispatch and cast back of
    a single row."""
    import combine_ep_layout_amd as ep
    from synth import Config, generate
    say(f"[fp8var] hidden 128 kind={kind} mn={mn}")
    cfg = Config("one_group", 9, 128, 1, 3, 3, 1)
    d = generate(cfg, 5)
    for ready in (False, True):
        h, pool, scales, L = _dispatch_check(cfg, d, kind, mn, tile_ready=ready)
        h.close()
    # one row cast back, MN-major with ld == rows
    q = pool[:1].contiguous()
    if mn:
        s1 = scales[:, :1].contiguous()
    else:
        s1 = scales[:1].contiguous()
    out = ep.cast_back(q, s1, kind, mn, rows=1)
    s_host = _scales_host(s1, np.zeros(1, np.uint32 if (mn and kind == "ue8m0") else np.uint8))
    assert np.array_equal(bits_of(out), oracle.cast_back(q.cpu().numpy(), s_host, kind, mn))
