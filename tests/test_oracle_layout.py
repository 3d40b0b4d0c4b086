"""Pins for the oracle's layout (CPU only).

The layout is a stable bucket sort of routing slots by expert with each bucket
padded to BLOCK_M rows (StreamEP README, "Streaming dispatch in one
paragraph"; blog "DeepEP MoE dispatch/combine", one DeepEP round).  The oracle
is pinned by: hand-worked cases, numpy's bincount and stable argsort (library
routines), the assignment-count invariant from the blog's correctness section
(N_valid,send = N_valid,recv = N_t * k), and brute force over every routing of
tiny shapes against an independent sorted() formulation.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from synth import CONFIGS, generate
from conftest import parse_golden, ints, rows_of


def _check_golden(case):
    idx = np.array(rows_of(case["topk_idx"]), dtype=np.int32)
    L = oracle.layout(idx, int(case["E"]), int(case["BM"]))
    assert L["expert_counts"].tolist() == ints(case["expert_counts"])
    assert L["expert_pool_block_offset"].tolist() == ints(case["expert_pool_block_offset"])
    assert L["num_tiles"] == int(case["num_tiles"])
    assert L["tile_expert"].tolist() == ints(case["tile_expert"])
    assert L["pool_arrival_target"].tolist() == ints(case["pool_arrival_target"])
    assert L["slot_to_pool_row"].tolist() == ints(case["slot_to_pool_row"])
    assert L["pool_recv_token"].tolist() == ints(case["pool_recv_token"])
    assert L["error"] == int(case["error"])


def test_golden_hand_worked(golden_dir):
    cases = parse_golden(os.path.join(golden_dir, "layout_hand.txt"))
    assert len(cases) >= 5
    for case in cases:
        _check_golden(case)


def test_empty_routing():
    idx = np.zeros((0, 4), np.int32)
    L = oracle.layout(idx, 5, 8)
    assert L["num_tiles"] == 0 and L["pool_rows"] == 0
    assert (L["expert_counts"] == 0).all() and (L["expert_pool_block_offset"] == 0).all()
    assert L["capacity_rows"] == 5 * 7 and (L["pool_recv_token"] == -1).all()


def _expected_by_argsort(idx, E, BM):
    """Independent construction from numpy's stable argsort and bincount."""
    T, K = idx.shape
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    tiles = -(-counts // BM)
    off = np.concatenate([[0], np.cumsum(tiles)])
    cap = T * K + E * (BM - 1)
    recv = np.full(cap, -1, np.int64)
    s2r = np.full(T * K, -1, np.int64)
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    order = order[: int(valid.sum())]          # valid slots, grouped by expert, slot-ascending
    start = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        sl = order[start[e]:start[e + 1]]
        rows = off[e] * BM + np.arange(len(sl))
        s2r[sl] = rows
        recv[rows] = sl // K
    return counts, off, recv, s2r


@pytest.mark.parametrize("name", ["tiny", "decode", "share", "prefill", "stream"])
def test_configs_against_numpy(name):
    cfg = CONFIGS[name]
    d = generate(cfg, 0)
    idx = d["topk_idx"]
    E, BM = cfg.num_experts, cfg.block_m
    L = oracle.layout(idx, E, BM)
    counts, off, recv, s2r = _expected_by_argsort(idx, E, BM)
    assert L["error"] == 0
    assert np.array_equal(L["expert_counts"], counts)
    assert np.array_equal(L["expert_pool_block_offset"], off)
    assert np.array_equal(L["pool_recv_token"], recv)
    assert np.array_equal(L["slot_to_pool_row"], s2r)
    # the assignment-count invariant: every unmasked slot is received once
    n_valid = int((idx >= 0).sum())
    assert int(L["expert_counts"].sum()) == n_valid
    assert int((L["pool_recv_token"] >= 0).sum()) == n_valid
    if cfg.local_keep is None and cfg.mask_frac == 0:
        assert n_valid == cfg.tokens * cfg.top_k
    _check_invariants(idx, E, BM, L)


def _check_invariants(idx, E, BM, L):
    T, K = idx.shape
    counts = L["expert_counts"].astype(np.int64)
    off = L["expert_pool_block_offset"].astype(np.int64)
    nt = L["num_tiles"]
    te, tt = L["tile_expert"], L["pool_arrival_target"]
    s2r, recv = L["slot_to_pool_row"], L["pool_recv_token"]
    assert off[0] == 0 and np.array_equal(np.diff(off), -(-counts // BM))
    assert nt == off[-1] and L["pool_rows"] == nt * BM
    # every tile belongs to one expert; targets are the real rows per tile
    for e in range(E):
        tiles = np.arange(off[e], off[e + 1])
        assert (te[tiles] == e).all()
        assert tt[tiles].sum() == counts[e]
        if len(tiles):
            assert (tt[tiles[:-1]] == BM).all() and 1 <= tt[tiles[-1]] <= BM
    assert (te[nt:] == -1).all() and (tt[nt:] == 0).all()
    # slot_to_pool_row is a bijection from unmasked slots onto real rows
    flat = idx.ravel()
    valid = flat >= 0
    rows = s2r[valid]
    assert (s2r[~valid] == -1).all()
    assert len(np.unique(rows)) == len(rows)
    assert np.array_equal(np.sort(rows), np.flatnonzero(recv >= 0))
    slots = np.flatnonzero(valid)
    assert np.array_equal(recv[rows], slots // K)
    # each real row sits in its expert's tile, and rows of an expert ascend in slot order
    assert np.array_equal(te[rows // BM], flat[valid])
    for e in range(E):
        se = np.flatnonzero(flat == e)
        assert np.all(np.diff(s2r[se]) == 1)
    # padding rows: inside [0, P) but beyond a tile's target, and all rows >= P
    r = np.arange(len(recv))
    tile = r // BM
    in_pool = tile < nt
    real = np.zeros(len(recv), bool)
    real[in_pool] = (r[in_pool] - tile[in_pool] * BM) < tt[tile[in_pool]]
    assert np.array_equal(real, recv >= 0)


def _brute(idx_rows, E, BM):
    """Layout of a tiny routing by sorted(): pool rows per expert in slot order."""
    K = len(idx_rows[0]) if idx_rows else 0
    slots = [(s, e) for s, e in enumerate(itertools.chain.from_iterable(idx_rows))]
    err = int(any(e < -1 or e >= E for _, e in slots))
    counts = [sum(1 for _, e in slots if e == x) for x in range(E)]
    off = [0]
    for c in counts:
        off.append(off[-1] + (c + BM - 1) // BM)
    s2r = {}
    for e in range(E):
        mine = sorted(s for s, x in slots if x == e)
        for i, s in enumerate(mine):
            s2r[s] = off[e] * BM + i
    s2r_list = [s2r.get(s, -1) for s in range(len(slots))]
    cap = len(slots) + E * (BM - 1)
    recv = [-1] * cap
    for s, r in s2r.items():
        recv[r] = s // K
    return counts, off, s2r_list, recv, err


def test_brute_force_all_tiny_routings():
    n = 0
    for T, K in [(1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2)]:
        for ids in itertools.product([-1, 0, 1, 2], repeat=T * K):
            rows = [list(ids[t * K:(t + 1) * K]) for t in range(T)]
            idx = np.array(rows, dtype=np.int32)
            for E in (3,):
                for BM in (1, 2, 3, 4):
                    L = oracle.layout(idx, E, BM)
                    counts, off, s2r, recv, err = _brute(rows, E, BM)
                    assert L["expert_counts"].tolist() == counts
                    assert L["expert_pool_block_offset"].tolist() == off
                    assert L["slot_to_pool_row"].tolist() == s2r
                    assert L["pool_recv_token"].tolist() == recv
                    assert L["error"] == err
                    n += 1
    assert n == 4 * (4 + 16 + 16 + 256 + 64 + 4096)


def test_brute_force_out_of_range_ids():
    # E = 2: id 2 and id -2 are outside [-1, E) and must be flagged and skipped
    for ids in itertools.product([-2, -1, 0, 1, 2], repeat=4):
        rows = [list(ids[0:2]), list(ids[2:4])]
        idx = np.array(rows, dtype=np.int32)
        for BM in (1, 3):
            L = oracle.layout(idx, 2, BM)
            counts, off, s2r, recv, err = _brute(rows, 2, BM)
            assert L["expert_counts"].tolist() == counts
            assert L["slot_to_pool_row"].tolist() == s2r
            assert L["pool_recv_token"].tolist() == recv
            assert L["error"] == err


def test_skew_all_slots_one_expert():
    T, K, E, BM = 300, 3, 7, 16
    idx = np.full((T, K), 4, np.int32)
    L = oracle.layout(idx, E, BM)
    assert L["expert_counts"].tolist() == [0, 0, 0, 0, 900, 0, 0]
    assert L["num_tiles"] == 57 and L["pool_arrival_target"][56] == 900 - 56 * 16
    _check_invariants(idx, E, BM, L)
