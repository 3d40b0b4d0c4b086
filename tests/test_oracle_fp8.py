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
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    _, vals = _table()
    for e in (-127, -100, -9, 0, 7, 100):
        n = len(codes)
        H = 128 * ((n + 127) // 128)
        q = np.zeros(H, np.uint8)
        q[:n] = codes
        s = np.full(H // 128, e + 127, np.uint8)
        got = oracle.dequant_rows(q[None, :], s[None, :])[0][:n]
        mag = vals[codes & 0x7F] * 2.0 ** e
        want = bf16_from_f32(np.where(codes & 0x80, -mag, mag).astype(np.float32))
        assert np.array_equal(got, want), e


def test_quantize_roundtrip_on_e4m3_grid():
    # values already on the e4m3 grid times 2^e survive quantisation exactly
    _, vals = _table()
    x32 = np.concatenate([vals[::-1], -vals[1:]])[:128].astype(np.float32) * 2.0 ** -3
    x = bf16_from_f32(x32)
    q, s = oracle.quantize_row(x)
    assert int(s[0]) - 127 == -3
    assert np.array_equal(oracle.dequant_rows(q[None, :], s[None, :])[0], x)
