"""The oracle's results at full workload sizes: test infrastructure, used by
the GPU parity tests and by the benchmark's CPU-baseline leg only.

The oracle's per-token functions are called from a pool of host threads
(ctypes releases the interpreter lock during a foreign call, so the plain C
oracle runs on several cores).  Only the work is split, over tokens; every
value is the one the oracle computes for that token, and nothing here does
any of the method's arithmetic itself: dispatch results are the oracle's
per-token quantisation placed at the token's pool rows, as the dispatch
definition says (a token's codes and scales are computed once and written to
each of its rows)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Optional

import numpy as np

import oracle


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(n: int, parts: int):
    step = max(1, -(-n // parts))
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def _run(n: int, fn: Callable[[int, int], None], min_chunk: int = 64) -> None:
    parts = max(1, min(threads() * 4, n // min_chunk if n >= min_chunk else 1))
    with ThreadPoolExecutor(max_workers=threads()) as ex:
        for f in [ex.submit(fn, a, b) for a, b in _chunks(n, parts)]:
            f.result()


def quantize_tokens(x: np.ndarray, tokens: Optional[np.ndarray] = None, kind: str = "ue8m0"):
    """Per-token e4m3fn codes and per-128-channel scales of rows x[t] for t in
    `tokens` (default: every token): (codes [n, H] u8, scales [n, H/128]),
    u8 UE8M0 bytes or float32 for the float flavours."""
    tokens = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    n, H = tokens.size, x.shape[1]
    q = np.empty((n, H), np.uint8)
    s = np.empty((n, H // 128), np.uint8 if kind == "ue8m0" else np.float32)

    def work(a, b):
        for i in range(a, b):
            if kind == "f32":
                q[i], s[i] = oracle.quantize_row_f32scale(x[tokens[i]])
            else:
                q[i], e = oracle.quantize_row(x[tokens[i]])
                s[i] = e if kind == "ue8m0" else oracle.pow2_scales_from_ue8m0(e)

    _run(n, work, min_chunk=16)
    return q, s


def dequant_tokens(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """bf16(value(code) * 2^e) of UE8M0-scaled rows, row by row."""
    out = np.empty(q.shape, np.uint16)

    def work(a, b):
        out[a:b] = oracle.dequant_rows(q[a:b], s[a:b])

    _run(q.shape[0], work, min_chunk=16)
    return out


def combine(expert_out: np.ndarray, slot_to_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """oracle.combine over token ranges (each range reads its own slots' rows)."""
    T, K = weights.shape
    H = expert_out.shape[1]
    eo = np.ascontiguousarray(expert_out, dtype=np.uint16)
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    y = np.empty((T, H), np.uint16)

    def work(a, b):
        y[a:b] = oracle.combine(eo, s2r[a * K:b * K], weights[a:b])

    _run(T, work)
    return y


def combine_backward(grad_y: np.ndarray, expert_out: np.ndarray, slot_to_row: np.ndarray,
                     weights: np.ndarray, grad_eo: np.ndarray):
    """oracle.combine_backward over token ranges; the gradient rows are
    written into grad_eo (every range owns distinct rows).  Returns
    (grad_eo, grad_weights [T, K] float32)."""
    T, K = weights.shape
    eo = np.ascontiguousarray(expert_out, dtype=np.uint16)      # one copy at most, shared
    gy = np.ascontiguousarray(grad_y, dtype=np.uint16)
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    gw = np.empty((T, K), np.float32)

    def work(a, b):
        _, gw[a:b] = oracle.combine_backward(gy[a:b], eo, s2r[a * K:b * K],
                                             weights[a:b], grad_eo_out=grad_eo)

    _run(T, work)
    return grad_eo, gw


def dispatch_backward(grad_pool: np.ndarray, slot_to_row: np.ndarray, tokens: int,
                      top_k: int) -> np.ndarray:
    H = grad_pool.shape[1]
    gp = np.ascontiguousarray(grad_pool, dtype=np.uint16)
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    gx = np.empty((tokens, H), np.uint16)

    def work(a, b):
        gx[a:b] = oracle.dispatch_backward(gp, s2r[a * top_k:b * top_k], b - a, top_k)

    _run(tokens, work)
    return gx


def dispatch_bf16_rows(x: np.ndarray, recv_token: np.ndarray) -> np.ndarray:
    """oracle.dispatch_bf16 over ranges of pool rows (every range writes its own rows)."""
    recv = np.ascontiguousarray(recv_token, dtype=np.int32)
    pool = np.zeros((recv.size, x.shape[1]), np.uint16)

    def work(a, b):
        pool[a:b] = oracle.dispatch_bf16(x, recv[a:b])

    _run(recv.size, work, min_chunk=1024)
    return pool


def dispatch_fp8_rows(x: np.ndarray, recv_token: np.ndarray):
    """oracle.dispatch_fp8 over ranges of pool rows: the oracle quantises each
    row from its token, as it does in one call."""
    recv = np.ascontiguousarray(recv_token, dtype=np.int32)
    H = x.shape[1]
    pool = np.zeros((recv.size, H), np.uint8)
    scales = np.zeros((recv.size, H // 128), np.uint8)

    def work(a, b):
        pool[a:b], scales[a:b] = oracle.dispatch_fp8(x, recv[a:b])

    _run(recv.size, work, min_chunk=64)
    return pool, scales
