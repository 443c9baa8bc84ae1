"""Seeded synthetic inputs for the dispatch/combine path.

This module only draws inputs: the token rows ``x`` (bf16 bit patterns), the
routing ``topk_idx`` and the ``topk_weights``.  It holds none of the method's
arithmetic, and it is the one module that both the HIP path's tests/benchmark
and the CPU oracle's checks take their inputs from.

Workloads (all synthetic; the pages measure on no public dataset):

==========  ======  =====  ===  ===  ===  ===  =================================
name        tokens  hidden  R    E    k    C    routing
==========  ======  =====  ===  ===  ===  ===  =================================
tiny        64      256     8    16   2    4    uniform without replacement
sweep       128     7168    16   256  8    12   uniform
prefill     4096    7168    64   256  8    24   uniform
skew        4096    7168    32   256  8    24   Zipf(1.2) over a permutation, 10%
                                                 of slots masked to -1
large       16384   4096    16   64   6    32   uniform
==========  ======  =====  ===  ===  ===  ===  =================================

Draw order for one workload, from ``numpy.random.default_rng(seed)``:
  1. x = standard_normal((t, h), float32), rounded to bf16 (round to nearest even);
  2. Zipf only: perm = permutation(E); popularity of expert perm[i] is (i+1)^-s;
  3. topk_idx[t] = choice(E, k, replace=False[, p]) token by token (int64);
  4. masked workloads: floor(frac * t * k) distinct flat slots set to -1;
  5. logits = standard_normal((t, k)); weights = softmax over the valid slots of
     each token (float64, then float32); masked slots get weight 0.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    ranks: int
    experts: int
    topk: int
    channels: int
    routing: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 1.2
    mask_frac: float = 0.0
    seed: int = 0
    expert_alignment: int = 1

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 8, 16, 2, 4),
    "sweep": Workload("sweep", 128, 7168, 16, 256, 8, 12),
    "prefill": Workload("prefill", 4096, 7168, 64, 256, 8, 24),
    "skew": Workload("skew", 4096, 7168, 32, 256, 8, 24, routing="zipf", mask_frac=0.1),
    "large": Workload("large", 16384, 4096, 16, 64, 6, 32),
}


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) through torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def draw_x(rng: np.random.Generator, tokens: int, hidden: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((tokens, hidden), dtype=np.float32))


def draw_routing(rng: np.random.Generator, w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Returns (topk_idx int64 [t][k], topk_weights float32 [t][k])."""
    T, E, K = w.tokens, w.experts, w.topk
    p = None
    if w.routing == "zipf":
        perm = rng.permutation(E)
        p = np.empty(E, np.float64)
        p[perm] = (np.arange(E, dtype=np.float64) + 1.0) ** (-w.zipf_s)
        p /= p.sum()
    elif w.routing != "uniform":
        raise ValueError(f"unknown routing {w.routing!r}")
    idx = np.empty((T, K), np.int64)
    for t in range(T):
        idx[t] = rng.choice(E, K, replace=False, p=p)
    if w.mask_frac > 0.0:
        n_mask = int(np.floor(w.mask_frac * T * K))
        flat = rng.choice(T * K, n_mask, replace=False)
        idx.reshape(-1)[flat] = -1
    logits = rng.standard_normal((T, K))
    valid = idx >= 0
    logits = np.where(valid, logits, -np.inf)
    m = np.max(logits, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(logits - m), 0.0)
    s = e.sum(axis=1, keepdims=True)
    wts = np.where(s > 0, e / np.where(s > 0, s, 1.0), 0.0).astype(np.float32)
    return idx, wts


def generate(w: Workload | str, seed: int | None = None, with_x: bool = True) -> dict:
    """Draw one workload's inputs.  ``with_x=False`` skips x (routing-only checks)
    but keeps the draw order, so routing is identical either way."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if with_x:
        x = draw_x(rng, w.tokens, w.hidden)
    else:
        # advance the stream exactly as the x draw would
        rng.standard_normal((w.tokens, w.hidden), dtype=np.float32)
        x = None
    topk_idx, topk_weights = draw_routing(rng, w)
    return dict(workload=w, x=x, topk_idx=topk_idx, topk_weights=topk_weights)


def fp8_rows(x_bits: np.ndarray, block: int = 128) -> tuple[np.ndarray, np.ndarray]:
    """fp8 inputs of the fp8 dispatch workload, prepared the way a caller would
    (per token, per `block` elements: scale = amax / 448, element = x / scale
    cast to float8 e4m3 by torch).  Returns (uint8 bit patterns [t][h],
    float32 scales [t][h / block])."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).float()
    T, H = t.shape
    g = t.reshape(T, H // block, block)
    amax = g.abs().amax(dim=2, keepdim=True).clamp(min=1e-12)
    scale = amax / 448.0
    q = (g / scale).to(torch.float8_e4m3fn).reshape(T, H)
    return q.view(torch.uint8).numpy().copy(), scale.reshape(T, H // block).numpy().astype(np.float32).copy()

