"""GPU parity of dispatch (bf16 copy and FP8 e4m3fn + UE8M0) against the
oracle: pool and scale bytes bit-exact, padding rows never written."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Config, generate
from gpu_helpers import (say, inputs, oracle_layout, new_handle, device_routing, to_dev_bf16,
                         bits_of, full_path_check, dev, POISON_BF16, POISON_U8)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,tokens", [("tiny", -1), ("share", -1), ("prefill", 700),
                                         ("decode", 64)])
def test_bf16_full_compare(name, tokens):
    say(f"[dispatch bf16] {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    cfg = cfg.replace(fp8=False)
    full_path_check(cfg, d)


@pytest.mark.parametrize("name,tokens", [("decode", -1), ("stream", 2048)])
def test_fp8_full_compare(name, tokens):
    say(f"[dispatch fp8] {name} tokens={tokens}")
    cfg, d = inputs(name, tokens)
    full_path_check(cfg, d, fp8=True)


def _full_size_dispatch(name, fp8):
    """Every pool row (and FP8 scale row) of a full-size dispatch against the
    oracle: a real row holds its token's bytes, a padding row keeps its
    poison.  The oracle quantises each token once; its codes and scales are
    the expected contents of each of the token's rows."""
    from oracle import par as oracle_par
    cfg, d = inputs(name)
    L = oracle_layout(name)
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    cap, H = h.capacity_rows, cfg.hidden
    recv = L["pool_recv_token"]
    real = np.flatnonzero(recv >= 0)
    pad = np.flatnonzero(recv < 0)
    padt = torch.from_numpy(pad).to(dev())
    if fp8:
        pool = torch.full((cap, H), POISON_U8, dtype=torch.uint8, device=dev())
        scales = torch.full((cap, H // 128), POISON_U8, dtype=torch.uint8, device=dev())
        h.dispatch(x, pool, scales, fp8=True)
        q_tok, s_tok = oracle_par.quantize_tokens(d["x"])
        step = 32768
        for r0 in range(0, len(real), step):
            rows = real[r0:r0 + step]
            rt = torch.from_numpy(rows).to(dev())
            assert np.array_equal(pool[rt].cpu().numpy(), q_tok[recv[rows]]), r0
            assert np.array_equal(scales[rt].cpu().numpy(), s_tok[recv[rows]]), r0
        assert bool((pool[padt] == POISON_U8).all()) and bool((scales[padt] == POISON_U8).all())
        say(f"  {len(real)} rows of codes and scales match, {len(pad)} padding rows untouched")
    else:
        pool = torch.full((cap, H), POISON_BF16 - 0x10000, dtype=torch.int16,
                          device=dev()).view(torch.bfloat16)
        h.dispatch(x, pool)
        assert bool((pool.view(torch.int16)[padt] == POISON_BF16 - 0x10000).all())
        # every real row, on the device, against the row of x the oracle's
        # layout says it came from (the bf16 dispatch is a bitwise copy)
        realt = torch.from_numpy(real).to(dev())
        srct = torch.from_numpy(recv[real].astype(np.int64)).to(dev())
        assert torch.equal(pool.view(torch.int16)[realt], x.view(torch.int16)[srct])
        say(f"  {len(real)} rows match, {len(pad)} padding rows untouched")
    h.close()


@pytest.mark.parametrize("name,tokens,top_k,hidden", [("prefill", 8192, 1, 4096), ("prefill", 8192, 2, 4096),
                                                     ("prefill", 8192, 4, 4096), ("prefill", 8192, 8, 4096),
                                                     ("prefill", 8192, 3, 4224), ("prefill", 8192, 8, 4224),
                                                     ("share", 16384, 8, 2048)])
def test_bf16_dispatch_shapes_write_the_same_pool(name, tokens, top_k, hidden):
    """The bf16 dispatch's two launch shapes (a read pass over x, then one
    workgroup per token segment for dense routing; waves over tokens
    otherwise), each forced with the density hint on the same layout, against
    the oracle's layout: every real row is its token's row of x, every
    padding row keeps its poison.  8192 tokens x hidden 4096 (64 MiB of x,
    where the shape depends on the density), and hidden 4224, whose rows end
    in a partial segment; the share routing (about one real row per token)
    forced into the dense shape as well; then the shape the handle takes by
    itself, for this routing."""
    import combine_ep_layout_amd as ep
    say(f"[dispatch bf16] both launch shapes, {name} routing, {tokens} tokens, top_k={top_k}, hidden={hidden}")
    cfg = CONFIGS[name].replace(tokens=tokens, hidden=hidden, top_k=top_k)
    d = generate(cfg, 5)
    L = oracle.layout(d["topk_idx"], cfg.num_experts, cfg.block_m)
    recv = L["pool_recv_token"]
    real = torch.from_numpy(np.flatnonzero(recv >= 0)).to(dev())
    pad = torch.from_numpy(np.flatnonzero(recv < 0)).to(dev())
    src = torch.from_numpy(recv[recv >= 0].astype(np.int64)).to(dev())
    h = new_handle(cfg)
    h.layout(*device_routing(d))
    x = to_dev_bf16(d["x"])
    for hint in (ep.EP_DENSITY_DENSE, ep.EP_DENSITY_SPARSE, ep.EP_DENSITY_AUTO):
        h.set_density_hint(hint)
        pool = torch.full((h.capacity_rows, cfg.hidden), POISON_BF16 - 0x10000, dtype=torch.int16,
                          device=dev()).view(torch.bfloat16)
        h.dispatch(x, pool)
        torch.cuda.synchronize()
        assert torch.equal(pool.view(torch.int16)[real], x.view(torch.int16)[src]), hint
        assert bool((pool.view(torch.int16)[pad] == POISON_BF16 - 0x10000).all()), hint
        say(f"  hint {hint}: {real.numel()} rows match, {pad.numel()} padding rows untouched")
    assert h.sync_status() == ep.EP_OK
    h.close()


def test_bf16_prefill_full_size():
    say("[dispatch bf16] prefill full size")
    _full_size_dispatch("prefill", fp8=False)


def test_fp8_stream_full_size():
    say("[dispatch fp8] stream full size, every row")
    _full_size_dispatch("stream", fp8=True)


def _one_row_per_token(x_bits: np.ndarray) -> Config:
    T, H = x_bits.shape
    return Config("rows", T, H, 1, 1, 1, 1)


def test_fp8_every_bf16_pattern():
    """All 65536 bf16 bit patterns (NaN and infinities included) through the
    quantiser, in natural order, shuffled, and next to amax values that pin
    the scale exponent at the ends of its range."""
    say("[dispatch fp8] all bf16 patterns")
    H = 4096
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(7)
    rows = [allp.reshape(-1, H), rng.permutation(allp).reshape(-1, H)]
    # groups of 127 probes + one amax setter 448 * 2^e for e in a spread of exponents
    finite = allp[(allp & 0x7F80) != 0x7F80]
    for e in (-127, -126, -120, -9, -1, 0, 1, 60, 119):
        setter = np.array([0x43E0 + (e << 7)], np.uint16)   # bf16 pattern of 448 * 2^e
        mag = finite & 0x7FFF
        probes = finite[(mag <= setter[0]) & (mag > 0)]
        probes = rng.permutation(probes)[: 127 * 64]
        probes = np.resize(probes, 127 * 64).reshape(64, 127)
        groups = np.concatenate([np.repeat(setter[None, :], 64, 0), probes], axis=1)
        rows.append(groups.reshape(-1, H))
    x_bits = np.ascontiguousarray(np.concatenate(rows, axis=0))
    T = x_bits.shape[0]
    cfg = _one_row_per_token(x_bits)
    d = {"x": x_bits, "topk_idx": np.zeros((T, 1), np.int32),
         "topk_weights": np.ones((T, 1), np.float32)}
    full_path_check(cfg, d, fp8=True)


def test_fp8_nonfinite_inputs():
    say("[dispatch fp8] NaN / inf rows")
    H = 256
    rng = np.random.default_rng(2)
    x = rng.integers(0x3000, 0x4000, size=(6, H), dtype=np.uint16)
    x[0, 3] = 0x7FC0          # NaN: ignored by amax, code 0x7F
    x[1, 5] = 0xFFC1          # negative NaN
    x[2, 7] = 0x7F80          # +inf: scale 254, saturates to 0x7E
    x[3, 130] = 0xFF80        # -inf in the second group
    x[4, :128] = 0x0000       # all-zero group: scale byte 0
    x[5, :] = 0x8000          # negative zeros
    cfg = _one_row_per_token(x)
    d = {"x": x, "topk_idx": np.zeros((6, 1), np.int32), "topk_weights": np.ones((6, 1), np.float32)}
    full_path_check(cfg, d, fp8=True)


def test_fp8_every_scale_exponent():
    """Every UE8M0 exponent a finite group can take (e = -127 ... 120): for each,
    groups whose amax is 448 * 2^e (the largest finite bf16 for e = 120)
    holding every finite bf16 magnitude that fits under it, with random signs.
    The codes come from the hardware conversion where it applies, so this
    covers it over every (pattern, scale) pair the dispatch can meet."""
    say("[dispatch fp8] every scale exponent x every fitting magnitude")
    H = 4096
    rng = np.random.default_rng(11)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)                 # every finite nonzero magnitude
    rows = []
    for e in range(-127, 121):
        # amax 448 * 2^e; e = 120 is reached only by magnitudes above 448 * 2^119
        top = np.uint32(0x43E0 + (e << 7)) if e <= 119 else np.uint32(0x7F7F)
        fit = mags[mags <= top]
        fit = fit[fit != top]
        sgn = rng.integers(0, 2, size=fit.size, dtype=np.uint32) << 15
        probes = (fit | sgn).astype(np.uint16)
        ngroups = (probes.size + 126) // 127
        probes = np.resize(probes, ngroups * 127).reshape(ngroups, 127)
        groups = np.concatenate([np.full((ngroups, 1), top, np.uint16), probes], axis=1)
        flat = groups.reshape(-1)
        pad = (-flat.size) % H
        flat = np.concatenate([flat, np.zeros(pad, np.uint16)])
        rows.append(flat.reshape(-1, H))
    x_bits = np.ascontiguousarray(np.concatenate(rows, axis=0))
    T = x_bits.shape[0]
    say(f"  {T} tokens of hidden {H}")
    cfg = _one_row_per_token(x_bits)
    d = {"x": x_bits, "topk_idx": np.zeros((T, 1), np.int32),
         "topk_weights": np.ones((T, 1), np.float32)}
    full_path_check(cfg, d, fp8=True)
