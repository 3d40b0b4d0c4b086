"""CPU oracle for MoE EP dispatch/combine -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``ep_oracle.c`` (plain scalar C, built with gcc)
through ctypes and shares nothing with the HIP library.

Pinned functions (each checked in ``tests/test_oracle_*.py`` against something
other than itself): layout, bf16 dispatch, FP8 quantisation (scale exponent and
e4m3fn codes) in the UE8M0, float32 and power-of-two float32 scale flavours,
the MN-major and packed scale layouts, dequantisation (cast back), combine,
combine and dispatch backward.  Nothing here is "parity unpinned".
tests/test_oracle_mutants.py plants plausible mistakes in a copy of the C
source and checks that the pins reject every one.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libep_oracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.eo_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.eo_bf16_to_f32.restype = ctypes.c_float
    lib.eo_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.eo_f32_to_bf16.restype = ctypes.c_uint16
    lib.eo_e4m3_value.argtypes = [ctypes.c_int]
    lib.eo_e4m3_value.restype = ctypes.c_double
    lib.eo_e4m3_encode.argtypes = [ctypes.c_double]
    lib.eo_e4m3_encode.restype = ctypes.c_uint8
    lib.eo_ue8m0_exponent.argtypes = [ctypes.c_float]
    lib.eo_ue8m0_exponent.restype = ctypes.c_int
    lib.eo_quantize_row.argtypes = [P, ctypes.c_int32, P, P]
    lib.eo_quantize_row.restype = None
    lib.eo_dequant_row.argtypes = [P, P, ctypes.c_int32, P]
    lib.eo_dequant_row.restype = None
    lib.eo_layout.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                              ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P, P, P]
    lib.eo_layout.restype = ctypes.c_int64
    lib.eo_dispatch_bf16.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, P]
    lib.eo_dispatch_bf16.restype = None
    lib.eo_dispatch_fp8.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, P, P]
    lib.eo_dispatch_fp8.restype = None
    lib.eo_combine.argtypes = [P, ctypes.c_int32, P, P, ctypes.c_int64, ctypes.c_int32, P]
    lib.eo_combine.restype = None
    lib.eo_combine_gathered.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, P]
    lib.eo_combine_gathered.restype = None
    lib.eo_e4m3_encode_n.argtypes = [P, ctypes.c_int64, P]
    lib.eo_e4m3_encode_n.restype = None
    lib.eo_f32_to_bf16_n.argtypes = [P, ctypes.c_int64, P]
    lib.eo_f32_to_bf16_n.restype = None
    lib.eo_ue8m0_exponent_n.argtypes = [P, ctypes.c_int64, P]
    lib.eo_ue8m0_exponent_n.restype = None
    lib.eo_quantize_row_f32scale.argtypes = [P, ctypes.c_int32, P, P]
    lib.eo_quantize_row_f32scale.restype = None
    lib.eo_dequant_row_f32scale.argtypes = [P, P, ctypes.c_int32, P]
    lib.eo_dequant_row_f32scale.restype = None
    lib.eo_combine_backward.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, P, P]
    lib.eo_combine_backward.restype = None
    lib.eo_dispatch_backward.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P]
    lib.eo_dispatch_backward.restype = None
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def capacity_rows(tokens: int, top_k: int, num_experts: int, block_m: int) -> int:
    return tokens * top_k + num_experts * (block_m - 1)


# ------------------------------------------------------------- scalar forms --

def bf16_to_f32(b: int) -> float:
    return float(_load().eo_bf16_to_f32(int(b)))


def f32_to_bf16(f: float) -> int:
    return int(_load().eo_f32_to_bf16(float(f)))


def e4m3_value(code: int) -> float:
    return float(_load().eo_e4m3_value(int(code)))


def e4m3_encode(v: float) -> int:
    return int(_load().eo_e4m3_encode(float(v)))


def ue8m0_exponent(amax: float) -> int:
    return int(_load().eo_ue8m0_exponent(float(amax)))


# -------------------------------------------------------------- array forms --

def e4m3_encode_n(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _load().eo_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def f32_to_bf16_n(f: np.ndarray) -> np.ndarray:
    shape = np.shape(f)
    f = np.ascontiguousarray(f, dtype=np.float32).ravel()
    out = np.empty(f.size, dtype=np.uint16)
    _load().eo_f32_to_bf16_n(_p(f), f.size, _p(out))
    return out.reshape(shape)


def ue8m0_exponent_n(amax: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float32).ravel()
    out = np.empty(a.size, dtype=np.int32)
    _load().eo_ue8m0_exponent_n(_p(a), a.size, _p(out))
    return out


def quantize_row(x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.size
    q = np.empty(H, dtype=np.uint8)
    s = np.empty(H // 128, dtype=np.uint8)
    _load().eo_quantize_row(_p(x_row), H, _p(q), _p(s))
    return q, s


def quantize_row_f32scale(x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.size
    q = np.empty(H, dtype=np.uint8)
    s = np.empty(H // 128, dtype=np.float32)
    _load().eo_quantize_row_f32scale(_p(x_row), H, _p(q), _p(s))
    return q, s


def dequant_rows_f32scale(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    n, H = q.shape
    out = np.empty((n, H), dtype=np.uint16)
    lib = _load()
    for i in range(n):
        lib.eo_dequant_row_f32scale(_p(q[i]), _p(scales[i]), H, _p(out[i]))
    return out


# ------------------------------------------------------ scale formats -------
# The instagit page ("API Signature and Return Values") names three flavours
# of the per-128-channel scale: use_ue8m0 (a UE8M0 exponent byte), round_scale
# (a power-of-two scale kept as float32) and neither (a plain float32 scale).
# Readings where the page is silent: round_scale uses the UE8M0 exponent rule,
# so its codes equal the UE8M0 flavour's and its scale is the float 2^e; the
# GEMM-friendly "MN-major" layout stores group g of row r at [g, r] with a
# leading dimension ld >= rows, and UE8M0 bytes in that layout are packed four
# groups to a 32-bit word, group 4w + j in byte j of word w (unused bytes 0).

SCALE_UE8M0, SCALE_F32, SCALE_POW2_F32 = "ue8m0", "f32", "pow2_f32"


def pow2_scales_from_ue8m0(scale_bytes: np.ndarray) -> np.ndarray:
    """Float32 value 2^(byte - 127) of each UE8M0 byte (2^-127 is a float32 subnormal)."""
    e = scale_bytes.astype(np.int64) - 127
    return np.ldexp(np.float64(1.0), e).astype(np.float32)


def scale_words(groups: int) -> int:
    """32-bit words per row of packed UE8M0 scales."""
    return (groups + 3) // 4


def scales_to_mn_major(scales: np.ndarray, ld: int, init: Optional[np.ndarray] = None,
                       rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Row-major scales [n, G] -> MN-major.  float32 scales give float32 [G, ld];
    UE8M0 bytes give packed uint32 [ceil(G/4), ld].  Only the columns listed in
    `rows` (all n by default) are written; the rest keep `init` (zeros)."""
    n, G = scales.shape
    packed = scales.dtype == np.uint8
    nw = scale_words(G)
    shape = (nw, ld) if packed else (G, ld)
    dtype = np.uint32 if packed else np.float32
    out = np.zeros(shape, dtype) if init is None else np.array(init, dtype=dtype, copy=True)
    assert out.shape == shape
    rows = np.arange(n) if rows is None else rows
    for r in rows:
        if packed:
            for w in range(nw):
                word = 0
                for j in range(4):
                    g = 4 * w + j
                    if g < G:
                        word |= int(scales[r, g]) << (8 * j)
                out[w, r] = word
        else:
            out[:, r] = scales[r, :]
    return out


def scales_from_mn_major(mn: np.ndarray, n: int, groups: int) -> np.ndarray:
    """Inverse of scales_to_mn_major for the first n columns."""
    if mn.dtype == np.uint32:
        out = np.zeros((n, groups), np.uint8)
        for r in range(n):
            for g in range(groups):
                out[r, g] = (int(mn[g // 4, r]) >> (8 * (g % 4))) & 0xFF
        return out
    return np.ascontiguousarray(mn[:, :n].T.astype(np.float32))


def dispatch_fp8_scaled(x: np.ndarray, recv_token: np.ndarray, kind: str, mn_major: bool = False,
                        ld: Optional[int] = None, pool_init: Optional[np.ndarray] = None,
                        scales_init: Optional[np.ndarray] = None):
    """FP8 dispatch in any scale flavour and layout.  Real rows hold their
    token's codes and scales; padding rows (and MN-major columns past the pool)
    keep their initial contents."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    recv = np.ascontiguousarray(recv_token, dtype=np.int32)
    H = x.shape[1]
    G = H // 128
    cap = recv.size
    real = np.flatnonzero(recv >= 0)
    pool = (np.zeros((cap, H), np.uint8) if pool_init is None
            else np.array(pool_init, dtype=np.uint8, copy=True, order="C"))
    rm = np.zeros((cap, G), np.uint8 if kind == SCALE_UE8M0 else np.float32)
    for r in real:
        if kind == SCALE_F32:
            pool[r], rm[r] = quantize_row_f32scale(x[recv[r]])
        else:
            q, b = quantize_row(x[recv[r]])
            pool[r] = q
            rm[r] = b if kind == SCALE_UE8M0 else pow2_scales_from_ue8m0(b)
    if mn_major:
        scales = scales_to_mn_major(rm, ld if ld is not None else cap, scales_init, rows=real)
    else:
        scales = (np.zeros_like(rm) if scales_init is None
                  else np.array(scales_init, dtype=rm.dtype, copy=True, order="C"))
        scales[real] = rm[real]
    return pool, scales


def cast_back(q: np.ndarray, scales: np.ndarray, kind: str, mn_major: bool = False) -> np.ndarray:
    """bf16 rows from e4m3fn codes [n, H] and their scales (per_token_cast_back
    on the instagit page): UE8M0 and power-of-two scales are exact powers of
    two, float32 scales use one float product; both round once to bf16."""
    n, H = q.shape
    G = H // 128
    rm = scales_from_mn_major(scales, n, G) if mn_major else scales
    if kind == SCALE_UE8M0:
        return dequant_rows(q, rm)
    return dequant_rows_f32scale(q, rm.astype(np.float32))


def dequant_rows(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise rows q[n, H] with scales[n, H/128] to bf16 bits [n, H]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n, H = q.shape
    out = np.empty((n, H), dtype=np.uint16)
    lib = _load()
    for i in range(n):
        lib.eo_dequant_row(_p(q[i]), _p(scales[i]), H, _p(out[i]))
    return out


# ------------------------------------------------------------------ layout --

def layout(topk_idx: np.ndarray, num_experts: int, block_m: int,
           cap: Optional[int] = None) -> Dict[str, np.ndarray]:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    E, BM = int(num_experts), int(block_m)
    if cap is None:
        cap = capacity_rows(T, K, E, BM)
    max_tiles = cap // BM
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    num_tiles = np.zeros(1, np.int32)
    tile_expert = np.empty(max_tiles, np.int32)
    tile_target = np.empty(max_tiles, np.int32)
    slot_to_row = np.empty(T * K, np.int32)
    recv_token = np.empty(cap, np.int32)
    error = np.zeros(1, np.int32)
    P = _load().eo_layout(_p(idx), T, K, E, BM, cap, max_tiles, _p(counts), _p(offsets),
                          _p(num_tiles), _p(tile_expert), _p(tile_target), _p(slot_to_row),
                          _p(recv_token), _p(error))
    if P < 0:
        raise ValueError("pool capacity too small for this routing")
    return {"expert_counts": counts, "expert_pool_block_offset": offsets,
            "num_tiles": int(num_tiles[0]), "tile_expert": tile_expert,
            "pool_arrival_target": tile_target, "slot_to_pool_row": slot_to_row,
            "pool_recv_token": recv_token, "error": int(error[0]), "pool_rows": int(P),
            "capacity_rows": cap, "max_tiles": max_tiles}


# ---------------------------------------------------------------- dispatch --

def dispatch_bf16(x: np.ndarray, recv_token: np.ndarray,
                  pool_init: Optional[np.ndarray] = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    recv = np.ascontiguousarray(recv_token, dtype=np.int32)
    H = x.shape[1]
    cap = recv.size
    pool = (np.zeros((cap, H), np.uint16) if pool_init is None
            else np.array(pool_init, dtype=np.uint16, copy=True, order="C"))
    _load().eo_dispatch_bf16(_p(x), H, _p(recv), cap, _p(pool))
    return pool


def dispatch_fp8(x: np.ndarray, recv_token: np.ndarray, pool_init: Optional[np.ndarray] = None,
                 scales_init: Optional[np.ndarray] = None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    recv = np.ascontiguousarray(recv_token, dtype=np.int32)
    H = x.shape[1]
    cap = recv.size
    pool = (np.zeros((cap, H), np.uint8) if pool_init is None
            else np.array(pool_init, dtype=np.uint8, copy=True, order="C"))
    scales = (np.zeros((cap, H // 128), np.uint8) if scales_init is None
              else np.array(scales_init, dtype=np.uint8, copy=True, order="C"))
    _load().eo_dispatch_fp8(_p(x), H, _p(recv), cap, _p(pool), _p(scales))
    return pool, scales


# ----------------------------------------------------------------- combine --

def combine(expert_out: np.ndarray, slot_to_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    eo = np.ascontiguousarray(expert_out, dtype=np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    T, K = w.shape
    H = eo.shape[1]
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    y = np.empty((T, H), np.uint16)
    _load().eo_combine(_p(eo), H, _p(s2r), _p(w), T, K, _p(y))
    return y


def combine_gathered(rows: np.ndarray, valid: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """rows[n, K, H] bf16 bits, valid[n, K] (bool), weights[n, K] -> y[n, H]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    n, K, H = rows.shape
    v = np.ascontiguousarray(valid, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    y = np.empty((n, H), np.uint16)
    _load().eo_combine_gathered(_p(rows), _p(v), _p(w), n, K, H, _p(y))
    return y


# ---------------------------------------------------------------- backward --

def combine_backward(grad_y: np.ndarray, expert_out: np.ndarray, slot_to_row: np.ndarray,
                     weights: np.ndarray, grad_eo_init: Optional[np.ndarray] = None,
                     grad_eo_out: Optional[np.ndarray] = None):
    """Returns (grad_expert_out [cap, H] bf16 bits, grad_weights [T, K] float32).
    With grad_eo_out (a C-contiguous uint16 [cap, H] array) the gradient rows
    are written into it in place and it is returned; other rows keep its
    contents."""
    gy = np.ascontiguousarray(grad_y, dtype=np.uint16)
    eo = np.ascontiguousarray(expert_out, dtype=np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    T, K = w.shape
    H = gy.shape[1]
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    if grad_eo_out is not None:
        assert grad_eo_out.dtype == np.uint16 and grad_eo_out.flags["C_CONTIGUOUS"]
        assert grad_eo_out.shape == eo.shape
        geo = grad_eo_out
    else:
        geo = (np.zeros_like(eo) if grad_eo_init is None
               else np.array(grad_eo_init, dtype=np.uint16, copy=True, order="C"))
    gw = np.empty((T, K), np.float32)
    _load().eo_combine_backward(_p(gy), _p(eo), _p(s2r), _p(w), T, K, H, _p(geo), _p(gw))
    return geo, gw


def dispatch_backward(grad_pool: np.ndarray, slot_to_row: np.ndarray, tokens: int,
                      top_k: int) -> np.ndarray:
    gp = np.ascontiguousarray(grad_pool, dtype=np.uint16)
    H = gp.shape[1]
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    gx = np.empty((tokens, H), np.uint16)
    _load().eo_dispatch_backward(_p(gp), _p(s2r), tokens, top_k, H, _p(gx))
    return gx
