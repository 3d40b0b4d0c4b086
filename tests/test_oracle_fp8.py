"""Pins for the oracle's FP8 e4m3fn quantisation with UE8M0 scales (CPU only).

The payload format is torch.float8_e4m3fn with UE8M0 scales (instagit page,
"FP8 and Quantization Support").  Pins: hand-derived codes and scale bytes;
torch's CPU float32 -> float8_e4m3fn cast (a library routine) over every finite
bf16 pattern at several scale exponents; an independent nearest-value search
written with numpy; closed forms for the scale exponent; the quantisation
error bound; exact dequantisation.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f32, bf16_from_f32
from conftest import parse_golden


def _golden(golden_dir):
    codes, scales = [], []
    with open(os.path.join(golden_dir, "fp8_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, a, b = line.split()
            if kind == "code":
                codes.append((float(a), int(b, 16)))
            else:
                scales.append((float(a), int(b)))
    return codes, scales


def test_golden_codes_and_scales(golden_dir):
    codes, scales = _golden(golden_dir)
    assert len(codes) >= 20 and len(scales) >= 10
    for v, c in codes:
        assert oracle.e4m3_encode(v) == c, (v, hex(c))
    for amax, byte in scales:
        assert oracle.ue8m0_exponent(np.float32(amax)) + 127 == byte, (amax, byte)


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(b)
    return b[np.isfinite(f)], f[np.isfinite(f)]


def _torch_e4m3(v32):
    return torch.from_numpy(v32.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _table():
    codes = np.arange(0x7F)
    ef, m = codes >> 3, codes & 7
    vals = np.where(ef == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (ef.astype(np.float64) - 7))
    return codes, vals


def _nearest_search(v):
    """Independent e4m3fn encoder: distance to every finite code, ties to even."""
    codes, vals = _table()
    a = np.abs(v)[:, None]
    d = np.abs(a - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one
    pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 1 << 20).min(axis=1)
    single = np.where(cand, codes[None, :], 1 << 20).min(axis=1)
    code = np.where(cand.sum(axis=1) > 1, pick, single)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("e", [-127, -20, -7, 0, 5, 60])
def test_encode_matches_torch_cast_all_bf16(e):
    _, f = _all_finite_bf16()
    v = f.astype(np.float64) * 2.0 ** (-e)
    keep = np.abs(v) <= 448.0
    v = v[keep]
    got = oracle.e4m3_encode_n(v)
    want = _torch_e4m3(v.astype(np.float32))
    # float32 rounding of v can only matter below 2^-126, where every code is +-0
    assert np.array_equal(got, want)


@pytest.mark.parametrize("e", [-127, -8, 0, 3])
def test_encode_matches_nearest_search_all_bf16(e):
    _, f = _all_finite_bf16()
    v = f.astype(np.float64) * 2.0 ** (-e)
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle.e4m3_encode_n(v), _nearest_search(v))


def test_encode_midpoints_and_signed_zero():
    codes, vals = _table()
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.e4m3_encode_n(mids)
    lo = codes[:-1]
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode_n(-mids), (want | 0x80).astype(np.uint8))
    assert oracle.e4m3_encode(-0.0) == 0x80 and oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(float("inf")) == 0x7E and oracle.e4m3_encode(float("-inf")) == 0xFE


def test_scale_exponent_closed_form():
    _, f = _all_finite_bf16()
    a = np.abs(f[f != 0])
    e = oracle.ue8m0_exponent_n(a).astype(np.int64)
    assert e.min() >= -127 and e.max() <= 127
    r = a.astype(np.float64) * 2.0 ** (-e)
    clamped = e == -127
    # unclamped: the scaled amax lands in (224, 448] -- the smallest power of two that fits
    assert np.all((r[~clamped] > 224.0) & (r[~clamped] <= 448.0))
    assert np.all(r[clamped] <= 448.0)
    assert oracle.ue8m0_exponent(0.0) == -127


def test_quantize_row_error_bound_and_scale_rule():
    rng = np.random.default_rng(3)
    H = 512
    x32 = (rng.standard_normal(H) * np.repeat(2.0 ** rng.integers(-30, 30, H // 128), 128)).astype(np.float32)
    x = bf16_from_f32(x32)
    q, s = oracle.quantize_row(x)
    xf = bf16_to_f32(x).astype(np.float64)
    for g in range(H // 128):
        seg = xf[g * 128:(g + 1) * 128]
        e = int(s[g]) - 127
        amax = np.abs(seg).max()
        assert amax <= 448 * 2.0 ** e and (e == -127 or amax > 448 * 2.0 ** (e - 1))
    deq = bf16_to_f32(oracle.dequant_rows(q[None, :], s[None, :])[0]).astype(np.float64)
    e_c = np.repeat(s.astype(np.int64) - 127, 128)
    v = np.abs(xf) * 2.0 ** (-e_c)
    normal = v >= 2.0 ** -6
    # e4m3 keeps 3 mantissa bits: half-ulp relative error 2^-4 in the normal range,
    # and half the subnormal step 2^-10 (scaled) below it
    assert np.all(np.abs(deq - xf)[normal] <= 2.0 ** -4 * np.abs(xf)[normal])
    assert np.all(np.abs(deq - xf)[~normal] <= 2.0 ** (e_c[~normal] - 10))


def test_dequant_is_exact():
    """value(code) * 2^e for every non-NaN code; one row per exponent, all
    rows decoded in one call, so each row must take its own scales."""
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    _, vals = _table()
    exps = (-127, -100, -9, 0, 7, 100)
    n = len(codes)
    H = 128 * ((n + 127) // 128)
    q = np.zeros((len(exps), H), np.uint8)
    q[:, :n] = codes
    s = np.array([[e + 127] * (H // 128) for e in exps], np.uint8)
    got = oracle.dequant_rows(q, s)
    for i, e in enumerate(exps):
        mag = vals[codes & 0x7F] * 2.0 ** e
        want = bf16_from_f32(np.where(codes & 0x80, -mag, mag).astype(np.float32))
        assert np.array_equal(got[i][:n], want), e


def test_quantize_roundtrip_on_e4m3_grid():
    # values already on the e4m3 grid times 2^e survive quantisation exactly
    _, vals = _table()
    x32 = np.concatenate([vals[::-1], -vals[1:]])[:128].astype(np.float32) * 2.0 ** -3
    x = bf16_from_f32(x32)
    q, s = oracle.quantize_row(x)
    assert int(s[0]) - 127 == -3
    assert np.array_equal(oracle.dequant_rows(q[None, :], s[None, :])[0], x)


# ---------------------------------------------- float32-scale flavour -------
# Reading (the pages name use_ue8m0 = False without a rule): a = max(amax,
# 448 * 2^-126), s = a / 448, codes = e4m3fn(float(x * (448 / a))), all in
# float32.  Pinned against torch's float32 arithmetic and its float8_e4m3fn
# cast, and by the quantisation error bound.

FLOOR = np.float32(448.0) * np.float32(2.0 ** -126)


def _torch_f32scale(xf):
    a = np.maximum(np.where(np.isnan(xf), 0, np.abs(xf)).max(1), FLOOR).astype(np.float32)  # NaN takes no part
    s = (a / np.float32(448.0)).astype(np.float32)
    f = torch.from_numpy((np.float32(448.0) / a).astype(np.float32))
    v = torch.from_numpy(xf) * f[:, None]                    # float32 products
    nan = torch.isnan(v)
    v = torch.clamp(v.abs(), max=448.0)                      # torch's cast does not saturate
    q = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    q[nan.numpy()] = 0x7F
    q |= np.where(np.signbit(xf), 0x80, 0).astype(np.uint8)
    return q.ravel(), s


def test_f32scale_quantize_matches_torch():
    rng = np.random.default_rng(12)
    H = 1024
    for trial in range(24):
        x32 = (rng.standard_normal(H) * 2.0 ** rng.integers(-40, 40)).astype(np.float32)
        if trial == 0:
            x32[:128] = 0.0                     # an all-zero group: floor scale, codes +-0
            x32[64] = -0.0
        if trial == 1:
            x32[128:256] *= np.float32(2.0 ** -100)   # amax below the floor
            x32[300] = np.inf                   # an infinite amax: factor 0, inf * 0 is NaN
            x32[301] = np.nan
            x32[513] = -np.inf
        x = bf16_from_f32(x32)
        q, s = oracle.quantize_row_f32scale(x)
        want_q, want_s = _torch_f32scale(bf16_to_f32(x).reshape(-1, 128))
        assert np.array_equal(s, want_s)
        assert np.array_equal(q, want_q), trial


def test_f32scale_dequant_and_error_bound():
    rng = np.random.default_rng(13)
    H = 512
    x = bf16_from_f32(rng.standard_normal(H).astype(np.float32))
    q, s = oracle.quantize_row_f32scale(x)
    deq = oracle.dequant_rows_f32scale(q[None, :], s[None, :])[0]
    val = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float()
    want = (val.reshape(-1, 128) * torch.from_numpy(s)[:, None]).reshape(-1).to(torch.bfloat16)
    assert np.array_equal(deq, want.view(torch.int16).numpy().view(np.uint16))
    xf = bf16_to_f32(x).astype(np.float64)
    df = bf16_to_f32(deq).astype(np.float64)
    s_c = np.repeat(s.astype(np.float64), 128)
    normal = np.abs(xf) / s_c >= 2.0 ** -6
    # e4m3 half-ulp 2^-4 relative, the bf16 half-ulp 2^-9, float roundings
    assert np.all(np.abs(df - xf)[normal] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(xf)[normal])
    assert np.all(np.abs(df - xf)[~normal] <= 2.0 ** -10 * s_c[~normal] * 1.01 + 2.0 ** -8 * np.abs(xf)[~normal])
    # NaN codes come back as quiet NaNs with their sign
    nanq = np.array([0x7F, 0xFF] + [0] * 126, np.uint8)
    back = oracle.dequant_rows_f32scale(nanq[None, :], np.ones((1, 1), np.float32))[0]
    assert back[0] == 0x7FC0 and back[1] == 0xFFC0
    # a zero code times an infinite scale (a group whose amax was infinite)
    zq = np.array([0x00, 0x80, 0x38] + [0] * 125, np.uint8)
    back = oracle.dequant_rows_f32scale(zq[None, :], np.full((1, 1), np.inf, np.float32))[0]
    assert back[0] == 0x7FC0 and back[1] == 0xFFC0 and back[2] == 0x7F80      # 1.0 * inf = inf


# ------------------------------------------- power-of-two float32 scales ----

def test_pow2_scale_closed_form_and_codes():
    """round_scale without UE8M0: s = 2^e with e = ceil(log2(amax / 448)) in
    [-127, 127] (closed form via frexp), codes = torch's cast of x * 2^-e."""
    rng = np.random.default_rng(14)
    H = 1024
    x32 = (rng.standard_normal(H) * np.repeat(2.0 ** rng.integers(-135, 120, H // 128), 128)).astype(np.float32)
    x32[:128] = 0.0
    x = bf16_from_f32(x32)
    recv = np.array([0], np.int32)
    pool, s = oracle.dispatch_fp8_scaled(x[None, :], recv, oracle.SCALE_POW2_F32)
    xf = bf16_to_f32(x).reshape(-1, 128).astype(np.float64)
    amax = np.abs(xf).max(1)
    m, ex = np.frexp(amax / 448.0)                        # amax/448 exact in float64
    e = np.where(m == 0.5, ex - 1, ex)                    # ceil(log2(.)) of m * 2^ex
    e = np.clip(np.where(amax == 0, -127, e), -127, 127)
    assert np.array_equal(s[0], np.ldexp(1.0, e).astype(np.float32))
    v = (xf * np.ldexp(1.0, -e)[:, None]).astype(np.float32)   # exact power-of-two scaling
    assert np.array_equal(pool[0], _torch_e4m3(v.ravel()))


# ----------------------------------------------------- MN-major layouts ------

def test_mn_major_layouts_by_memory_view():
    """MN-major float scales are the transpose; packed UE8M0 words, read as
    little-endian bytes, are the row's group bytes four at a time."""
    rng = np.random.default_rng(15)
    n, G, ld = 7, 11, 12
    b = rng.integers(0, 256, size=(n, G), dtype=np.uint8)
    words = oracle.scales_to_mn_major(b, ld)
    assert words.shape == (3, ld) and words.dtype == np.uint32
    as_bytes = words.astype("<u4").view(np.uint8).reshape(3, ld, 4)     # [w, r, j]
    want = np.zeros((n, 12), np.uint8)
    want[:, :G] = b
    assert np.array_equal(as_bytes[:, :n, :].transpose(1, 0, 2).reshape(n, 12), want)
    assert (words[:, n:] == 0).all()
    assert np.array_equal(oracle.scales_from_mn_major(words, n, G), b)
    f = rng.standard_normal((n, G)).astype(np.float32)
    mn = oracle.scales_to_mn_major(f, ld)
    assert np.array_equal(mn[:, :n], f.T) and (mn[:, n:] == 0).all()
    assert np.array_equal(oracle.scales_from_mn_major(mn, n, G), f)


def test_scaled_dispatch_untouched_rows_and_cast_back():
    rng = np.random.default_rng(16)
    T, H = 5, 384
    x = bf16_from_f32((rng.standard_normal((T, H)) * 3).astype(np.float32))
    recv = np.array([2, -1, 0, 4, -1, 1, 3, -1], np.int32)
    real = recv >= 0
    for kind in (oracle.SCALE_UE8M0, oracle.SCALE_F32, oracle.SCALE_POW2_F32):
        p_rm, s_rm = oracle.dispatch_fp8_scaled(x, recv, kind)
        for mn in (False, True):
            packed = mn and kind == oracle.SCALE_UE8M0
            shape = ((1, 9) if packed else (3, 9)) if mn else (8, 3)
            init = np.full(shape, 0xA5A5A5A5 if packed else 0xA5,
                           np.uint32 if packed else (np.uint8 if kind == "ue8m0" else np.float32))
            p, s = oracle.dispatch_fp8_scaled(x, recv, kind, mn, ld=9, pool_init=np.full((8, H), 0x5A, np.uint8),
                                              scales_init=init)
            assert np.array_equal(p[real], p_rm[real]) and (p[~real] == 0x5A).all()
            if mn:
                cols = np.flatnonzero(real)
                assert np.array_equal(oracle.scales_from_mn_major(s, 8, 3)[real], s_rm[real])
                untouched = np.setdiff1d(np.arange(9), cols)
                assert np.array_equal(s[:, untouched], init[:, untouched])
            else:
                assert np.array_equal(s[real], s_rm[real]) and np.array_equal(s[~real], init[~real])
            back = oracle.cast_back(p[real], s_rm[real], kind)
            # the error bound ties the three flavours to the source rows
            src = bf16_to_f32(x[recv[real]]).astype(np.float64)
            got = bf16_to_f32(back).astype(np.float64)
            assert np.all(np.abs(got - src) <= 2.0 ** -4 * np.abs(src) + 2.0 ** -9 * np.abs(src) +
                          np.abs(src).max(1, keepdims=True) * 2.0 ** -15)
    # UE8M0 and power-of-two float scales decode to the same rows
    p8, s8 = oracle.dispatch_fp8_scaled(x, recv, oracle.SCALE_UE8M0)
    p2, s2 = oracle.dispatch_fp8_scaled(x, recv, oracle.SCALE_POW2_F32)
    assert np.array_equal(p8, p2)
    assert np.array_equal(oracle.cast_back(p8[real], s8[real], "ue8m0"),
                          oracle.cast_back(p2[real], s2[real], "pow2_f32"))
