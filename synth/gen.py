"""Seeded synthetic workloads for one GPU's share of MoE EP dispatch/combine.

The five named workloads follow the shapes and value distributions of the
DeepEP / StreamEP pages: bf16 activations x[num_tokens, hidden] ~ N(0, 1),
router output topk_idx[num_tokens, top_k] (-1 marks a masked slot) and
topk_weights[num_tokens, top_k] (softmax of N(0, 1) logits over the k slots).
The pages print no dataset; PR #769 on DeepEP measures on "deterministic,
fixed-route" synthetic routing, so seeded synthetic routing is the workload.

Draw order (part of the recipe, numpy PCG64 ``default_rng(seed)``):
  1. x      = bf16(standard_normal((T, H), float32))      (torch RNE cast)
  2. routing: uniform -> scores = random((T, E_global)); topk = stable argsort
              of -scores, first K columns (K distinct experts per token);
              zipf    -> perm = permutation(E); logp[perm[i]] = -s*ln(i+1);
              topk of logp + gumbel((T, E)) (sampling K distinct experts
              without replacement from a truncated Zipf(s) law).
  3. masking: local_keep  -> ids >= local_keep become -1 (one rank's share);
              mask_frac   -> random((T, K)) < mask_frac become -1.
  4. weights = float32(softmax over K of float64(standard_normal((T, K), f32))).
Expert outputs come from a separate stream ``default_rng([seed, 7])`` so that
drawing them never perturbs x or the routing.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    tokens: int
    hidden: int
    top_k: int
    num_experts: int          # experts handed to the library (local experts)
    experts_global: int       # experts the router draws from
    block_m: int
    routing: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 1.2
    local_keep: Optional[int] = None   # keep ids < local_keep, mask the rest
    mask_frac: float = 0.0
    fp8: bool = False
    tile_ready: bool = False
    expert: str = "normal"    # "normal": N(0,1) rows; "scale": x*(e+1)/8

    @property
    def slots(self) -> int:
        return self.tokens * self.top_k

    @property
    def capacity_rows(self) -> int:
        return self.tokens * self.top_k + self.num_experts * (self.block_m - 1)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 128, 256, 2, 8, 8, 16, expert="scale"),
    "decode": Config("decode", 256, 7168, 8, 64, 64, 64, fp8=True),
    "share": Config("share", 8192, 3072, 8, 16, 128, 128, local_keep=16),
    "prefill": Config("prefill", 16384, 7168, 8, 256, 256, 128, routing="zipf"),
    "stream": Config("stream", 32768, 4096, 8, 128, 128, 128, mask_frac=0.05,
                     fp8=True, tile_ready=True),
}


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), using torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 4096) -> np.ndarray:
    rows = shape[0]
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_from_f32(rng.standard_normal((r1 - r0,) + tuple(shape[1:]),
                                                       dtype=np.float32))
    return out


def _route(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    T, K = cfg.tokens, cfg.top_k
    if cfg.routing == "uniform":
        scores = rng.random((T, cfg.experts_global))
        idx = np.argsort(-scores, axis=1, kind="stable")[:, :K]
    elif cfg.routing == "zipf":
        E = cfg.experts_global
        perm = rng.permutation(E)
        logp = np.empty(E, dtype=np.float64)
        logp[perm] = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        g = rng.gumbel(size=(T, E))
        idx = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :K]
    else:
        raise ValueError(f"unknown routing {cfg.routing!r}")
    return np.ascontiguousarray(idx, dtype=np.int32)


def generate(cfg: Config, seed: int = 0) -> Dict[str, np.ndarray]:
    """Draw x (bf16 bits), topk_idx (int32) and topk_weights (float32)."""
    rng = np.random.default_rng(seed)
    T, H, K = cfg.tokens, cfg.hidden, cfg.top_k
    x = _normal_bf16(rng, (T, H))
    idx = _route(cfg, rng) if T > 0 else np.zeros((0, K), np.int32)
    if cfg.local_keep is not None:
        idx[idx >= cfg.local_keep] = -1
    if cfg.mask_frac > 0.0:
        m = rng.random((T, K)) < cfg.mask_frac
        idx[m] = -1
    logits = rng.standard_normal((T, K), dtype=np.float32).astype(np.float64)
    if T > 0:
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
    else:
        p = logits
    w = np.ascontiguousarray(p.astype(np.float32))
    return {"x": x, "topk_idx": idx, "topk_weights": w}


def expert_rows(tokens: int, top_k: int, hidden: int, seed: int = 0) -> np.ndarray:
    """Per-slot expert outputs o[t, k, :] as bf16 bits, ~ N(0, 1)."""
    rng = np.random.default_rng([seed, 7])
    out = np.empty((tokens, top_k, hidden), dtype=np.uint16)
    step = max(1, (1 << 22) // max(1, top_k * hidden))
    for t0 in range(0, tokens, step):
        t1 = min(tokens, t0 + step)
        out[t0:t1] = bf16_from_f32(rng.standard_normal((t1 - t0, top_k, hidden),
                                                       dtype=np.float32))
    return out
