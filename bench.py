"""Benchmark: one GPU's share of MoE EP dispatch + combine on MI355X.

A step is one pass of the whole path over one batch: layout (counts, scan,
tiles, stable ranks), dispatch (pool copy; FP8 quantisation and streaming
release where the workload asks for them) and combine.  The default workload
is the prefill share: 16384 tokens, hidden 7168, 256 experts with Zipf(1.2)
top-8 routing, BLOCK_M 128, bf16.  Inputs are seeded synthetic data already
resident in HBM when the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                    [--no-cpu-baseline] [--copy-calibration]
                    [--borrow-compare | --backward | --gate | --fp8-variants | --graph | --ceiling
                     | --overlap]

Prints one JSON line.  "value" is algorithmic bytes moved per step / step
time, over exactly K steps with nothing else on the stream.  Per-kernel times
(and the roofline's achieved bandwidth) come from a second timed pass of K
steps with HIP events recorded around every launch on the stream the kernels
are launched on (torch's current stream, which is passed to the library).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0     # MI355X HBM3E peak, GB/s
METRIC = "dispatch+combine HBM GB/s and % of MI355X peak; tokens/s at 16384 tok"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, idx: np.ndarray, counts: np.ndarray, fp8: bool):
    """Bytes each kernel must move, every item once (padding rows never move).

    layout:   read topk_idx + topk_weights, write slot_to_pool_row + weights
              (16*T*K) and pool_recv_token for every capacity row (4*cap)
    dispatch: read slot_to_pool_row (4*T*K), read each active token's row of
              x once (2*H*T_act), write N_a pool rows (b*H*N_a, b = 2 bf16 /
              1 fp8) and, for FP8, N_a*H/128 scale bytes
    combine:  read slot_to_pool_row + weights (8*T*K), read N_a expert rows
              (2*H*N_a), write y (2*H*T)
    """
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    valid = idx >= 0
    n_a = int(valid.sum())
    t_act = int(valid.any(1).sum())
    cap = cfg.capacity_rows
    b = 1 if fp8 else 2
    layout = 16 * T * K + 4 * cap
    dispatch = 4 * T * K + 2 * H * t_act + b * H * n_a + (n_a * (H // 128) if fp8 else 0)
    combine = 8 * T * K + 2 * H * n_a + 2 * H * T
    return {"layout": layout, "dispatch": dispatch, "combine": combine,
            "n_a": n_a, "t_act": t_act, "pool_rows": int(((counts + cfg.block_m - 1)
                                                          // cfg.block_m).sum() * cfg.block_m)}


def kernel_source_sha() -> str:
    """Hash of the library sources with comments and blank space removed, so
    that a comment edit does not orphan counters taken on the same code."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_ep_layout_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "ep_ceiling.hip":                    # the bandwidth probes, not the path
            continue
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode())
        h.update(text.encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, per_launch_alg: float):
    """HBM traffic of a kernel from the committed rocprofv3 counter summary,
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, d, eo_host: np.ndarray, reps: int, tokens: int):
    """Time the oracle on the first `tokens` tokens of the same workload (all
    of them when tokens >= T), twice: as it stands, on one host thread, and
    with its dispatch and combine split over token or row ranges on every
    host core this process may use (at most 16), calling the same oracle
    functions; the layout is a global stable sort and runs on one thread in
    both.  GB/s uses the same algorithmic byte counts as the GPU figure, for
    that sample."""
    import oracle
    from oracle import par
    n = min(tokens, cfg.tokens)
    sub = {k: v[:n] for k, v in d.items()}
    scfg = cfg.replace(tokens=n)
    L0 = oracle.layout(sub["topk_idx"], cfg.num_experts, cfg.block_m)
    ab = algorithmic_bytes(scfg, sub["topk_idx"], L0["expert_counts"], cfg.fp8)
    alg = ab["layout"] + ab["dispatch"] + ab["combine"]

    def leg(threaded: bool):
        times, stages = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            L = oracle.layout(sub["topk_idx"], cfg.num_experts, cfg.block_m)
            t1 = time.perf_counter()
            if cfg.fp8:
                (par.dispatch_fp8_rows if threaded else oracle.dispatch_fp8)(sub["x"], L["pool_recv_token"])
            else:
                (par.dispatch_bf16_rows if threaded else oracle.dispatch_bf16)(sub["x"], L["pool_recv_token"])
            t2 = time.perf_counter()
            (par.combine if threaded else oracle.combine)(eo_host, L["slot_to_pool_row"], sub["topk_weights"])
            t3 = time.perf_counter()
            times.append(t3 - t0)
            stages.append((t1 - t0, t2 - t1, t3 - t2))
        t = float(np.median(times))
        st = np.median(np.array(stages), axis=0)
        return {"value": round(alg / t / 1e9, 3), "unit": "GB/s",
                "cores": par.threads() if threaded else 1,
                "seconds_per_pass": round(t, 3),
                "stage_seconds": {"layout": round(float(st[0]), 4),
                                  "dispatch": round(float(st[1]), 4),
                                  "combine": round(float(st[2]), 4)}}

    one = leg(False)
    many = leg(True)
    what = (f"the full {cfg.name} workload ({n} tokens)" if n == cfg.tokens else
            f"the first {n} of {cfg.tokens} tokens of the {cfg.name} workload")
    out = dict(many)
    out.update({"kind": "oracle", "tokens": n, "tokens_per_s": round(n / many["seconds_per_pass"], 1),
                "sample": f"{what}, layout + dispatch + combine, median of {reps} passes; dispatch and "
                          f"combine split over {many['cores']} host threads (layout on one)",
                "single_thread": one})
    return out


def borrow_compare(steps: int, warmup: int) -> dict:
    """Borrowed receive view vs copying dispatch, each followed by the same
    indexed consumer (the tile consumer stand-in reading every real row), at
    the per-GPU shape of DeepEP PR #769: hidden 3072, top-8, 16 local of 128
    experts, 1024 / 8192 / 16384 tokens."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import CONFIGS, generate
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    rows = []
    for T in (1024, 8192, 16384):
        cfg = CONFIGS["share"].replace(tokens=T)
        d = generate(cfg, 0)
        H = cfg.hidden
        idx = torch.from_numpy(d["topk_idx"]).to(dev)
        w = torch.from_numpy(d["topk_weights"]).to(dev)
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
        h = ep.EpHandle(T, cfg.top_k, cfg.num_experts, cfg.block_m)
        pool, _ = h.new_pool(H)
        out = torch.empty(h.capacity_rows, H, dtype=torch.bfloat16, device=dev)
        wg = h.max_tiles

        def copy_path():
            h.layout(idx, w)
            h.dispatch(x, pool)
            h.tile_consume(0, pool, None, H, out, workgroups=wg)

        def borrow_path():
            h.layout(idx, w)
            h.borrow(x)
            h.tile_consume(0, x, None, H, out, workgroups=wg, gather=True)
            h.release()

        res = {}
        for name, fn in (("copy", copy_path), ("borrow", borrow_path), ("copy2", copy_path),
                         ("borrow2", borrow_path)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            res[name] = a.elapsed_time(b) / steps * 1e3
        assert h.sync_status() == ep.EP_OK
        h.close()
        c = min(res["copy"], res["copy2"])
        bo = min(res["borrow"], res["borrow2"])
        rows.append({"tokens": T, "copy_us": round(c, 2), "borrow_us": round(bo, 2),
                     "change_pct": round(100.0 * (bo - c) / c, 1)})
    return {"metric": "borrowed receive view vs copying dispatch, each with the same indexed "
                      "consumer (layout + dispatch + consumer time)",
            "unit": "us", "higher_is_better": False, "data": "synthetic",
            "config": {"workload": "hidden 3072, top-8, 16 local of 128 experts, BLOCK_M 128, bf16"},
            "results": rows,
            "pages_context": "8xH200, hidden 3072, top-8, 16 local experts: -13.1% at 8192 "
                             "tokens/rank, -13.5% at 16384, +15.9% at 1024"}


def backward_bench(cfg, steps: int, warmup: int) -> dict:
    """Times combine_grads and dispatch_grads on one workload.  Algorithmic
    bytes: combine backward reads grad_y (2HT), the expert rows (2H*N_a) and
    the slot map + weights (8TK), writes the gradient rows (2H*N_a) and grad_w
    (4TK); dispatch backward reads the gradient rows (2H*N_a) and the slot map
    (4TK) and writes grad_x (2HT)."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    epoch = h.layout(idx, w)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    eo = torch.empty(h.capacity_rows, H, dtype=torch.bfloat16, device=dev)
    for r0 in range(0, h.capacity_rows, 16384):
        r1 = min(h.capacity_rows, r0 + 16384)
        eo[r0:r1] = torch.randn(r1 - r0, H, generator=g, device=dev).to(torch.bfloat16)
    gy = torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)
    geo = torch.empty_like(eo)
    gw = torch.empty(T, K, dtype=torch.float32, device=dev)
    gx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        ep.ep_combine_backward(h.raw, epoch, gy, eo, geo, gw)
        ep.ep_dispatch_backward(h.raw, epoch, geo, gx)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        ep.ep_combine_backward(h.raw, epoch, gy, eo, geo, gw)
        e[1].record(stream)
        ep.ep_dispatch_backward(h.raw, epoch, geo, gx)
        e[2].record(stream)
    torch.cuda.synchronize()
    cb = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    db = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    assert h.sync_status() == ep.EP_OK
    h.close()
    n_a = int((d["topk_idx"] >= 0).sum())
    b_cb = 2 * H * T + 4 * H * n_a + 12 * T * K
    b_db = 2 * H * n_a + 4 * T * K + 2 * H * T
    return {"metric": "combine_grads + dispatch_grads HBM GB/s", "unit": "GB/s",
            "value": round((b_cb + b_db) / ((cb + db) * 1e-6) / 1e9, 2), "higher_is_better": True,
            "data": "synthetic", "dtype": "bf16",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}"},
            "kernels_us": {"combine_backward": round(cb, 2), "dispatch_backward": round(db, 2)},
            "alg_bytes": {"combine_backward": b_cb, "dispatch_backward": b_db},
            "gbs": {"combine_backward": round(b_cb / (cb * 1e-6) / 1e9, 1),
                    "dispatch_backward": round(b_db / (db * 1e-6) / 1e9, 1)},
            "pct_of_peak": round(100.0 * (b_cb + b_db) / ((cb + db) * 1e-6) / 1e9 / PEAK_GBS, 2)}


def _time_us(fn, steps: int, warmup: int, stream) -> float:
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1e3


def _time_in_step_us(before, fn, after, steps: int, warmup: int, stream, flush=None) -> float:
    """Mean duration of fn's launches when each one runs between `before` and
    `after` (the kernels around it in a step), from HIP events on `stream`;
    with `flush`, it runs before every timed step."""
    import torch
    for _ in range(warmup):
        before()
        fn()
        after()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        if flush is not None:
            flush()
        before()
        a.record(stream)
        fn()
        b.record(stream)
        after()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3


def graph_bench(cfg, steps: int, warmup: int, per_replay: int = 4, separate: bool = False) -> dict:
    """The layout -> dispatch -> combine step launched eagerly vs captured in
    a HIP graph of `per_replay` steps (torch's graph capture on the library's
    stream).  Small batches are launch-bound, and a graph replay removes the
    gaps between launches.  Batches of at most 2048 slots take the one-launch
    ep_layout_dispatch unless `separate`.  The graph's output is checked
    against the eager step's."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    dev = torch.device("cuda", 0)
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    fp8, ready = cfg.fp8, cfg.tile_ready
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    pool, scales = h.new_pool(H, fp8=fp8)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    eo = torch.randn(h.capacity_rows, H, generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    one_launch = not ready and T * K <= 2048 and not separate

    def step():
        if one_launch:
            e, _ = h.layout_dispatch(idx, w, x, pool, scales, fp8=fp8)
        else:
            e = h.layout(idx, w)
            h.dispatch(x, pool, scales, fp8=fp8, tile_ready=ready)
        h.combine(e, eo, y)

    s = torch.cuda.Stream()                              # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eager = _time_us(step, steps, warmup, s)
        want = y.clone()
        # a captured combine cannot wait for its layout's density report:
        # fix its launch shape to the density the eager layouts reported
        density = h.layout_density(s)
        h.set_density_hint(density)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for _ in range(per_replay):
                step()
        torch.cuda.synchronize()
        y.zero_()
        n = max(1, steps // per_replay)
        replay = _time_us(graph.replay, n, max(1, warmup // per_replay), s) / per_replay
    torch.cuda.synchronize()
    same = bool(torch.equal(y.view(torch.int16), want.view(torch.int16)))
    status = h.sync_status()
    del graph
    h.close()
    if not same or status != ep.EP_OK:
        raise RuntimeError("graph replay differs from the eager step")
    return {"metric": "layout+dispatch+combine step, eager vs captured in a HIP graph",
            "unit": "us", "higher_is_better": False, "data": "synthetic",
            "dtype": "fp8" if fp8 else "bf16",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}, "
                                   f"{'fp8' if fp8 else 'bf16'}" + (", tile_ready" if ready else ""),
                       "steps_per_replay": per_replay},
            "step_calls": "ep_layout_dispatch, ep_combine" if one_launch else "ep_layout, ep_dispatch, ep_combine",
            "combine_density_hint": {1: "sparse", 2: "dense"}.get(density, "auto"),
            "eager_us_per_step": round(eager, 2), "graph_us_per_step": round(replay, 2),
            "change_pct": round(100.0 * (replay - eager) / eager, 1),
            "graph_output_equals_eager": same}


def gate_bench(cfg, steps: int, warmup: int, serial: bool = False) -> dict:
    """Per-token combine gate.  (1) The gate's own cost: the gated combine
    with every token already done vs the plain combine.  (2) A forward pass
    layout -> dispatch (tile_ready) -> expert-output producer (the tile
    consumer stand-in, copying each tile to expert_out and signalling its
    tokens) -> combine, once in order on one stream with the plain combine,
    once with the producer on a second stream overlapping the dispatch and
    the gated combine on a third overlapping the producer.  With `serial`
    (for counter passes, which run one kernel at a time) only (1) runs."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    dev = torch.device("cuda", 0)
    sa = torch.cuda.current_stream()
    sb, sc = torch.cuda.Stream(), torch.cuda.Stream()          # default priority
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    pool, _ = h.new_pool(H)
    eo = torch.zeros(h.capacity_rows, H, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    wg = 256
    spin = 2_000_000
    # (1) gate cost with all tokens done
    epoch = h.layout(idx, w)
    seq = h.dispatch(x, pool, tile_ready=True)
    h.tile_consume(seq, pool, None, H, eo, workgroups=wg, spin_limit_us=spin, signal_done=True)
    torch.cuda.synchronize()
    plain = _time_us(lambda: h.combine(epoch, eo, y), steps, warmup, sa)
    gated = _time_us(lambda: h.combine_gated(epoch, eo, 1, y, spin), steps, warmup, sa)

    # (2) forward pass, in order vs overlapped
    def in_order():
        ep_ = h.layout(idx, w)
        s = h.dispatch(x, pool, tile_ready=True)
        h.tile_consume(s, pool, None, H, eo, workgroups=wg, spin_limit_us=spin, signal_done=True)
        h.combine(ep_, eo, y)

    def overlapped():
        ep_ = h.layout(idx, w)
        e0 = torch.cuda.Event()
        e0.record(sa)
        sb.wait_event(e0)
        s = h.dispatch(x, pool, tile_ready=True, stream=sa)
        h.tile_consume(s, pool, None, H, eo, workgroups=wg, spin_limit_us=spin, signal_done=True,
                       stream=sb)
        e1 = torch.cuda.Event()
        e1.record(sa)
        sc.wait_event(e1)
        h.combine_gated(ep_, eo, 1, y, spin, stream=sc)
        e2 = torch.cuda.Event()
        e2.record(sc)
        e3 = torch.cuda.Event()
        e3.record(sb)
        sa.wait_event(e2)
        sa.wait_event(e3)

    if serial:
        t_order = t_over = t_order2 = t_over2 = float("nan")
    else:
        t_order = _time_us(in_order, steps, warmup, sa)
        t_over = _time_us(overlapped, steps, warmup, sa)
        t_order2 = _time_us(in_order, steps, warmup, sa)
        t_over2 = _time_us(overlapped, steps, warmup, sa)
    assert h.sync_status() == ep.EP_OK
    h.close()
    n_a = int((d["topk_idx"] >= 0).sum())
    comb_bytes = 8 * T * K + 2 * H * n_a + 2 * H * T
    if serial:
        return {"metric": "gated combine with every token done (serial run)", "unit": "us",
                "combine_us": round(plain, 2), "combine_gated_all_done_us": round(gated, 2)}
    return {"metric": "per-token combine gate: gate cost and forward pass with overlap",
            "unit": "us", "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}",
                       "producer_workgroups": wg},
            "combine_us": round(plain, 2), "combine_gated_all_done_us": round(gated, 2),
            "gate_cost_pct": round(100.0 * (gated - plain) / plain, 2),
            "combine_gated_gbs": round(comb_bytes / (gated * 1e-6) / 1e9, 1),
            "forward_in_order_us": round(min(t_order, t_order2), 2),
            "forward_overlapped_us": round(min(t_over, t_over2), 2),
            "overlap_change_pct": round(100.0 * (min(t_over, t_over2) - min(t_order, t_order2))
                                        / min(t_order, t_order2), 2)}


def fp8_variants_bench(cfg, steps: int, warmup: int) -> dict:
    """FP8 dispatch in every scale flavour and layout, and the cast back of
    the used pool rows.  Dispatch bytes as in the main benchmark (scale bytes
    1 per group for UE8M0, 4 for float32); cast back reads P rows of codes and
    their scales and writes P bf16 rows (P = used pool rows).  The dispatch is
    timed inside the layout -> dispatch -> combine step, as in the main
    benchmark: timed back to back on its own, the scale array would stay in
    the caches between calls, which hides what partial-line scale writes cost
    in a pipeline.  The cast back is timed back to back."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    G = H // 128
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    h.layout(idx, w)
    counts, nt = h.counts_to_host()
    P = nt * cfg.block_m
    valid = d["topk_idx"] >= 0
    n_a = int(valid.sum())
    t_act = int(valid.any(1).sum())
    out = torch.empty(P, H, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    eo = torch.randn(h.capacity_rows, H, generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    state = {}

    def before():
        state["epoch"] = h.layout(idx, w)

    def after():
        h.combine(state["epoch"], eo, y)

    combos = [(kind, mn) for kind in ("ue8m0", "f32", "pow2_f32") for mn in (False, True)]
    pools = {c: h.new_pool(H, fp8=True, scale_kind=c[0], mn_major=c[1]) for c in combos}
    best = {}
    for rep in range(2):                  # two passes over every combination, best of each
        for kind, mn in combos:
            pool, scales = pools[(kind, mn)]
            t_d = _time_in_step_us(before, lambda: h.dispatch(x, pool, scales, fp8=True,
                                                              scale_kind=kind, mn_major=mn),
                                   after, steps, warmup, stream)
            t_c = _time_us(lambda: ep.cast_back(pool, scales, kind, mn, rows=P, out=out),
                           steps, warmup, stream)
            o = best.get((kind, mn), (1e18, 1e18))
            best[(kind, mn)] = (min(o[0], t_d), min(o[1], t_c))
    rows = []
    for kind, mn in combos:
        t_d, t_c = best[(kind, mn)]
        sb = 1 if kind == "ue8m0" else 4
        b_d = 4 * T * K + 2 * H * t_act + H * n_a + sb * G * n_a
        b_c = P * H + sb * G * P + 2 * H * P
        rows.append({"scales": kind, "mn_major": mn,
                     "dispatch_us": round(t_d, 2), "dispatch_gbs": round(b_d / (t_d * 1e-6) / 1e9, 1),
                     "cast_back_us": round(t_c, 2), "cast_back_gbs": round(b_c / (t_c * 1e-6) / 1e9, 1)})
    assert h.sync_status() == ep.EP_OK
    h.close()
    return {"metric": "FP8 dispatch and cast back per scale flavour and layout", "unit": "us",
            "higher_is_better": False, "data": "synthetic", "dtype": "fp8 e4m3fn",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}",
                       "pool_rows_cast_back": P},
            "results": rows}


def overlap_bench(cfg, steps: int, warmup: int, workgroups: int = 256) -> dict:
    """Streaming dispatch on one stream and the tile consumer stand-in on a
    second stream, enqueued right after it (StreamEP README: a consumer spins
    on tile_ready and starts while later tokens are still landing).  HIP
    events give each kernel's interval; the consumer's acquire stamps (device
    wall clock, and whether its first look found the tile not ready) show how
    many tiles it took while the dispatch was still running, and the rank
    correlation of their acquire times with the last token each tile holds
    shows that tiles were released in token order.  The same two kernels run
    back to back on one stream for comparison."""
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    dev = torch.device("cuda", 0)
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()                                   # default priority
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    fp8 = cfg.fp8
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    pool, scales = h.new_pool(H, fp8=fp8)
    out = torch.empty(h.capacity_rows, H, dtype=torch.bfloat16, device=dev)
    spin = 2_000_000
    recv = None
    rows = []
    for it in range(warmup + steps):
        h.layout(idx, w)
        e = torch.cuda.Event()
        e.record(sa)
        sb.wait_event(e)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(sa)
        seq = h.dispatch(x, pool, scales, fp8=fp8, tile_ready=True, stream=sa)
        ev[1].record(sa)
        ev[2].record(sb)
        h.tile_consume(seq, pool, scales, H, out, fp8=fp8, workgroups=workgroups,
                       spin_limit_us=spin, stream=sb, stamps=True)
        ev[3].record(sb)
        sa.wait_stream(sb)
        torch.cuda.synchronize()
        if it < warmup:
            continue
        if h.sync_status() != ep.EP_OK:
            raise RuntimeError("a consumer wait timed out")
        nt = int(h.array("num_tiles").cpu()[0])
        if recv is None:
            recv = h.array("pool_recv_token").cpu().numpy()
            last_tok = np.array([recv[j * cfg.block_m:(j + 1) * cfg.block_m].max() for j in range(nt)])
        st = h.array("tile_stamp").cpu().numpy().view(np.uint64)[:nt]
        waited = (st >> np.uint64(63)).astype(bool)
        clock = (st & np.uint64((1 << 63) - 1)).astype(np.int64)
        t = [0.0] + [ev[0].elapsed_time(e_) * 1e3 for e_ in ev[1:]]
        rho = None
        if waited.sum() >= 2:
            ra = np.argsort(np.argsort(clock[waited])).astype(np.float64)
            rb = np.argsort(np.argsort(last_tok[waited])).astype(np.float64)
            ra -= ra.mean()
            rb -= rb.mean()
            rho = float((ra * rb).sum() / np.sqrt((ra * ra).sum() * (rb * rb).sum()))
        rows.append({"dispatch_us": t[1], "consumer_start_us": t[2], "consumer_end_us": t[3],
                     "overlap_us": max(0.0, min(t[1], t[3]) - max(0.0, t[2])),
                     "tiles": nt, "tiles_taken_while_landing": int(waited.sum()),
                     "rank_corr_acquire_vs_last_token": rho})

    def in_order():
        h.layout(idx, w)
        s_ = h.dispatch(x, pool, scales, fp8=fp8, tile_ready=True)
        h.tile_consume(s_, pool, scales, H, out, fp8=fp8, workgroups=workgroups, spin_limit_us=spin)

    def overlapped():
        h.layout(idx, w)
        e = torch.cuda.Event()
        e.record(sa)
        sb.wait_event(e)
        s_ = h.dispatch(x, pool, scales, fp8=fp8, tile_ready=True, stream=sa)
        h.tile_consume(s_, pool, scales, H, out, fp8=fp8, workgroups=workgroups,
                       spin_limit_us=spin, stream=sb)
        sa.wait_stream(sb)

    t_order = _time_us(in_order, steps, warmup, sa)
    t_over = _time_us(overlapped, steps, warmup, sa)
    if h.sync_status() != ep.EP_OK:
        raise RuntimeError("a consumer wait timed out")
    h.close()
    med = {k: float(np.median([r[k] for r in rows])) for k in
           ("dispatch_us", "consumer_start_us", "consumer_end_us", "overlap_us")}
    return {"metric": "streaming dispatch with the tile consumer on a second stream: overlap",
            "unit": "us", "higher_is_better": False, "data": "synthetic",
            "dtype": "fp8" if fp8 else "bf16",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}, "
                                   f"{'fp8' if fp8 else 'bf16'}, tile_ready",
                       "consumer_workgroups": workgroups},
            "median_us_from_dispatch_start": {k: round(v, 2) for k, v in med.items()},
            "per_rep": rows,
            "layout_dispatch_consumer_in_order_us": round(t_order, 2),
            "layout_dispatch_consumer_two_streams_us": round(t_over, 2)}


def ceiling_bench(cfg, steps: int, warmup: int) -> dict:
    """Context for the roofline: what simple HBM-bound kernels reach on this
    GPU, measured with the probe library (libep_ceiling.so: rows of 2*hidden
    bytes moved in 16-byte accesses by one wave per row, "@1w", by a
    256-thread workgroup per row, "@4w", or by one wave per 1 KB piece of a
    row, one access per lane, "@piece"), on the workload's own row size and
    row count N_a (every routed slot's row once):

      flat_write*       the same bytes as one flat array, every thread striding
                        over it (non-temporal or plain stores)
      seq_*             rows 0..N_a-1 in order (write, plain-store write, read,
                        copy)
      dispatch_order_*  the pool rows of the workload's layout in slot order,
                        as dispatch writes them and combine reads them
      pool_order_write  the same rows sorted by pool row
      random_write      the same rows in a seeded random order

    beside the library's own dispatch (bf16) and combine on the same layout,
    and torch's fill_ / copy_ over 2 GiB.  These are measured ceilings of
    plain kernels, not the nameplate peak."""
    import ctypes
    import torch
    import combine_ep_layout_amd as ep
    from synth import generate
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_ep_layout_amd", "libep_ceiling.so"))
    lib.ep_ceiling_rows.restype = ctypes.c_int
    lib.ep_ceiling_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    cap = h.capacity_rows
    epoch = h.layout(idx, w)
    s2r = h.array("slot_to_pool_row").cpu().numpy().reshape(-1)
    rows_slot = s2r[s2r >= 0].astype(np.int32)
    n_a = len(rows_slot)
    row_bytes = 2 * H
    perm = np.random.default_rng(0).permutation(n_a)
    orders = {"seq": np.arange(n_a, dtype=np.int32), "dispatch_order": rows_slot,
              "pool_order": np.sort(rows_slot), "random": rows_slot[perm]}
    orders = {k: torch.from_numpy(v).to(dev) for k, v in orders.items()}
    pool = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    pool.fill_(1.0)
    src = torch.ones(n_a, H, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(n_a, dtype=torch.int32, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)
    W, WD, R, C, WP, F, FP = 0, 1, 2, 3, 4, 5, 6

    def probe(op, wpr, rows, n_dst, dst=None, source=None):
        def fn():
            rc = lib.ep_ceiling_rows(op, wpr, None if dst is None else P(dst),
                                     None if source is None else P(source), n_dst, row_bytes,
                                     P(rows), n_a, P(sink), sp)
            if rc != 0:
                raise RuntimeError(f"ep_ceiling_rows returned {rc}")
        return fn

    nb = row_bytes * n_a
    legs = {"flat_write": (probe(F, 1, orders["seq"], n_a, dst=src), nb),
            "flat_write_plain": (probe(FP, 1, orders["seq"], n_a, dst=src), nb)}
    for wpr, tag in ((0, "piece"), (1, "1w"), (4, "4w")):
        for name, fn, nbytes in (
                ("seq_write", probe(W, wpr, orders["seq"], n_a, dst=src), nb),
                ("seq_write_plain", probe(WP, wpr, orders["seq"], n_a, dst=src), nb),
                ("seq_read", probe(R, wpr, orders["seq"], n_a, source=src), nb),
                ("seq_copy", probe(C, wpr, orders["seq"], cap, dst=pool, source=src), 2 * nb),
                ("dispatch_order_write", probe(W, wpr, orders["dispatch_order"], cap, dst=pool), nb),
                ("dispatch_order_write_device_scope",
                 probe(WD, wpr, orders["dispatch_order"], cap, dst=pool), nb),
                ("pool_order_write", probe(W, wpr, orders["pool_order"], cap, dst=pool), nb),
                ("random_write", probe(W, wpr, orders["random"], cap, dst=pool), nb),
                ("dispatch_order_read", probe(R, wpr, orders["dispatch_order"], cap, source=pool), nb)):
            legs[f"{name}@{tag}"] = (fn, nbytes)
    ab = algorithmic_bytes(cfg, d["topk_idx"], h.array("expert_counts").cpu().numpy(), False)
    lp, _ = h.new_pool(H)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    legs["library_dispatch_bf16"] = (lambda: h.dispatch(x, lp, None), ab["dispatch"])
    legs["library_combine"] = (lambda: h.combine(epoch, pool, y), ab["combine"])
    res = {}
    for name, (fn, nbytes) in legs.items():
        t = min(_time_us(fn, steps, warmup, stream) for _ in range(2))
        res[name] = {"us": round(t, 1), "GB_s": round(nbytes / (t * 1e-6) / 1e9, 1),
                     "frac_of_8TBs": round(nbytes / (t * 1e-6) / 1e9 / PEAK_GBS, 4)}
    assert h.sync_status() == ep.EP_OK
    h.close()
    del pool, src, lp
    n = 1 << 29                                          # 2 GiB of float32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for name, fn, nbytes in (("torch_fill", lambda: b.fill_(3.0), 4 * n),
                             ("torch_copy", lambda: b.copy_(a), 8 * n)):
        t = min(_time_us(fn, steps, warmup, stream) for _ in range(2))
        res[name] = {"us": round(t, 1), "GB_s": round(nbytes / (t * 1e-6) / 1e9, 1),
                     "frac_of_8TBs": round(nbytes / (t * 1e-6) / 1e9 / PEAK_GBS, 4)}
    del a, b
    return {"metric": "HBM bandwidth of plain kernels (context for the roofline)",
            "unit": "GB/s", "data": "synthetic",
            "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                                   f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}",
                       "rows": n_a, "row_bytes": row_bytes},
            "results": res}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the launch-bound tiny and decode workloads)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=None,
                    help="oracle passes, median taken (default 3 for prefill and stream, 11 otherwise)")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the CPU-oracle sample (default: all for bf16, 1024 for FP8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--borrow-compare", action="store_true",
                    help="print the borrowed-view vs copy comparison instead")
    ap.add_argument("--backward", action="store_true",
                    help="print the backward (combine_grads + dispatch_grads) measurement instead")
    ap.add_argument("--gate", action="store_true",
                    help="print the per-token combine gate measurement instead")
    ap.add_argument("--fp8-variants", action="store_true",
                    help="print the FP8 scale flavour / cast back measurement instead")
    ap.add_argument("--graph", action="store_true",
                    help="print the eager vs HIP-graph step time instead")
    ap.add_argument("--ceiling", action="store_true",
                    help="print the bandwidth of plain torch fill / read / copy kernels instead")
    ap.add_argument("--serial", action="store_true",
                    help="with --gate: skip the legs that need kernels running at the same time "
                         "(for counter passes, which serialise kernels)")
    ap.add_argument("--separate", action="store_true",
                    help="run layout and dispatch as two calls also where the one-launch "
                         "ep_layout_dispatch applies (batches of at most 2048 slots)")
    ap.add_argument("--overlap", action="store_true",
                    help="print the streaming dispatch / tile consumer overlap measurement instead "
                         "(default workload: stream)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 200 if args.config in ("tiny", "decode") else 20
    if args.cpu_reps is None:
        args.cpu_reps = 3 if args.config in ("prefill", "stream") else 11

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of EP dispatch/combine; runs on more than "
              "one GPU are not supported (use --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import combine_ep_layout_amd as ep
    from synth import CONFIGS, generate

    if args.copy_calibration:
        # a plain 1 GiB device copy, three times: the reference launch that
        # HBM counter passes scale their FETCH_SIZE / WRITE_SIZE by
        torch.cuda.set_device(0)
        a = torch.empty(1 << 29, dtype=torch.int16, device=torch.device("cuda", 0))
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.borrow_compare:
        torch.cuda.set_device(0)
        print(json.dumps(borrow_compare(args.steps, args.warmup)), flush=True)
        return 0
    if args.backward:
        torch.cuda.set_device(0)
        print(json.dumps(backward_bench(CONFIGS[args.config], args.steps, args.warmup)), flush=True)
        return 0
    if args.gate:
        torch.cuda.set_device(0)
        print(json.dumps(gate_bench(CONFIGS[args.config], args.steps, args.warmup, args.serial)),
              flush=True)
        return 0
    if args.graph:
        torch.cuda.set_device(0)
        print(json.dumps(graph_bench(CONFIGS[args.config], args.steps, args.warmup,
                                     separate=args.separate)), flush=True)
        return 0
    if args.ceiling:
        torch.cuda.set_device(0)
        print(json.dumps(ceiling_bench(CONFIGS[args.config], args.steps, args.warmup)), flush=True)
        return 0
    if args.overlap:
        torch.cuda.set_device(0)
        name = "stream" if args.config == "prefill" else args.config
        print(json.dumps(overlap_bench(CONFIGS[name], args.steps, args.warmup)), flush=True)
        return 0
    if args.fp8_variants:
        torch.cuda.set_device(0)
        print(json.dumps(fp8_variants_bench(CONFIGS[args.config], args.steps, args.warmup)),
              flush=True)
        return 0

    cfg = CONFIGS[args.config]
    fp8, ready = cfg.fp8, cfg.tile_ready
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    log(f"[bench] generating {cfg.name} inputs")
    d = generate(cfg, 0)
    T, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)

    h = ep.EpHandle(T, K, cfg.num_experts, cfg.block_m)
    cap = h.capacity_rows
    pool, scales = h.new_pool(H, fp8=fp8)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    eo = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    for r0 in range(0, cap, 16384):                       # chunked to bound the fp32 temporary
        r1 = min(cap, r0 + 16384)
        eo[r0:r1] = torch.randn(r1 - r0, H, generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # Batches of at most 2048 slots take the library's one-launch layout and
    # dispatch (ep_layout_dispatch) unless --separate asks for the two calls.
    one_launch = not ready and T * K <= 2048 and not args.separate
    phases = ("layout_dispatch", "combine") if one_launch else ("layout", "dispatch", "combine")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if one_launch:
            epoch, _ = h.layout_dispatch(idx, w, x, pool, scales, fp8=fp8)
        else:
            epoch = h.layout(idx, w)
            if ev is not None:
                ev[1].record(stream)
            h.dispatch(x, pool, scales, fp8=fp8, tile_ready=ready)
        if ev is not None:
            ev[len(phases) - 1].record(stream)
        h.combine(epoch, eo, y)
        if ev is not None:
            ev[len(phases)].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert h.sync_status() == ep.EP_OK

    def pct(v):
        return {"p10": round(float(np.percentile(v, 10)), 2), "p50": round(float(np.median(v)), 2),
                "p90": round(float(np.percentile(v, 90)), 2)}

    # Caches are flushed before every timed step: reading 1 GiB replaces L2
    # and the 256 MB MALL with clean lines (a read, not a write, so no dirty
    # line is left to be written back inside the timed kernels; the smaller
    # workloads would otherwise stay in the MALL from one step to the next).
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def do_flush():
        torch.sum(flush, dim=0, dtype=torch.int64, out=sink)

    do_flush()                                            # the fill's dirty lines go out here
    torch.cuda.synchronize()

    # Timed region (the headline): exactly K steps, each after a flush, with
    # a HIP event pair around the step only (the flush is outside it).
    log(f"[bench] timing {args.steps} steps, caches flushed before each")
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for a_, b_ in step_ev:
        do_flush()
        a_.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_us = np.array([a_.elapsed_time(b_) for a_, b_ in step_ev]) * 1e3
    ms_per_step = float(step_us.mean()) / 1e3

    # Per-kernel durations in flushed steps: a second pass of K steps with HIP
    # events around every launch, on the stream the library launches on.
    log(f"[bench] timing {args.steps} flushed steps per kernel")
    nev = len(phases) + 1
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for i in range(args.steps):
        do_flush()
        step(cold[i])
    torch.cuda.synchronize()
    cold_s = {k: np.array([e[j].elapsed_time(e[j + 1]) for e in cold]) * 1e3
              for j, k in enumerate(phases)}
    cold_ms = {k: float(v.mean()) / 1e3 for k, v in cold_s.items()}

    # Warm steps, labelled as such: K steps back to back between two events
    # (each step finds what the previous one left in L2 and MALL), then a pass
    # with events around every launch.
    log(f"[bench] timing {args.steps} warm steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    warm_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    warm_s = {k: np.array([e[j].elapsed_time(e[j + 1]) for e in evs]) * 1e3
              for j, k in enumerate(phases)}

    # With the streaming release on, the same dispatch without it, for
    # comparison, timed the same way: inside the layout -> dispatch -> combine
    # step, with HIP events around each dispatch.
    no_ready = no_ready_warm = None
    if ready:
        st = {}

        def before():
            st["epoch"] = h.layout(idx, w)

        def after():
            h.combine(st["epoch"], eo, y)

        def plain():
            h.dispatch(x, pool, scales, fp8=fp8, tile_ready=False)

        no_ready = _time_in_step_us(before, plain, after, args.steps, args.warmup, stream,
                                    flush=do_flush)
        no_ready_warm = _time_in_step_us(before, plain, after, args.steps, args.warmup, stream)
    del flush, sink

    counts, _ = h.counts_to_host()
    ab = algorithmic_bytes(cfg, d["topk_idx"], counts, fp8)
    total = ab["layout"] + ab["dispatch"] + ab["combine"]
    value = total / (ms_per_step * 1e-3) / 1e9
    warm_value = total / (warm_ms_per_step * 1e-3) / 1e9
    if one_launch:
        kern = {"layout_dispatch": (cold_ms["layout_dispatch"], ab["layout"] + ab["dispatch"]),
                "combine": (cold_ms["combine"], ab["combine"])}
    else:
        kern = {"dispatch": (cold_ms["dispatch"], ab["dispatch"]), "combine": (cold_ms["combine"], ab["combine"])}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic(dom, cfg.name, dom_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        eo_host = eo.view(torch.int16).cpu().numpy().view(np.uint16)
        ntok = args.cpu_tokens if args.cpu_tokens > 0 else (1024 if fp8 else T)
        cpu = cpu_baseline(cfg, d, eo_host, args.cpu_reps, ntok)
        del eo_host

    if cpu is not None:
        # per stage: oracle seconds scaled to the whole workload (linear in
        # tokens for a sample) over the GPU kernel's seconds
        scale = T / cpu["tokens"]
        gpu_s = {k: v * 1e-3 for k, v in cold_ms.items()}

        def speedups(stage_s):
            if one_launch:
                stage_s = {"layout_dispatch": stage_s["layout"] + stage_s["dispatch"],
                           "combine": stage_s["combine"]}
            return {k: round(stage_s[k] * scale / gpu_s[k], 1) for k in gpu_s}

        cpu["speedup_per_stage"] = speedups(cpu["stage_seconds"])
        cpu["single_thread"]["speedup_per_stage"] = speedups(cpu["single_thread"]["stage_seconds"])
    mode = "fp8" if fp8 else "bf16"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mode,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {T} tokens, hidden {H}, {cfg.num_experts} experts "
                               f"{cfg.routing} top-{K}, BLOCK_M {cfg.block_m}, {mode}"
                               + (", tile_ready" if ready else ""),
                   "tokens": T, "hidden": H, "top_k": K, "num_experts": cfg.num_experts,
                   "block_m": cfg.block_m, "routing": cfg.routing},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "pct_of_peak": round(100.0 * value / PEAK_GBS, 2),
        "timing": "caches flushed (1 GiB read) before every step; mean of the K steps' HIP-event "
                  "intervals, the flush outside them",
        "step_us_percentiles": pct(step_us),
        "kernels_us": {k: round(v * 1e3, 2) for k, v in cold_ms.items()},
        "step_calls": "ep_layout_dispatch, ep_combine" if one_launch else "ep_layout, ep_dispatch, ep_combine",
        "kernels_us_percentiles": {k: pct(v) for k, v in cold_s.items()},
        "warm": {"what": "K steps back to back (each step finds the previous step's data in L2 "
                         "and MALL), one event pair around all of them; per-kernel times from a "
                         "pass with events around every launch",
                 "ms_per_step": round(warm_ms_per_step, 4),
                 "value": round(warm_value, 2),
                 "pct_of_peak": round(100.0 * warm_value / PEAK_GBS, 2),
                 "tokens_per_s": round(T / (warm_ms_per_step * 1e-3), 1),
                 "kernels_us": {k: round(float(v.mean()), 2) for k, v in warm_s.items()},
                 "kernels_us_percentiles": {k: pct(v) for k, v in warm_s.items()},
                 "dispatch_us_without_tile_ready": None if no_ready_warm is None
                 else round(no_ready_warm, 2)},
        "dispatch_us_without_tile_ready": None if no_ready is None else round(no_ready, 2),
        "alg_bytes": {k: ab[k] for k in ("layout", "dispatch", "combine")},
        "routing_stats": {"n_assign": ab["n_a"], "active_tokens": ab["t_act"],
                          "pool_rows": ab["pool_rows"], "max_expert_rows": int(counts.max())},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic,
                     "timing": f"mean of the kernel's HIP-event intervals over {args.steps} "
                               f"flushed steps (a second pass, events around every launch)"},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    h.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
