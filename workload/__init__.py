"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module only *draws* inputs: router logits with a Zipf-shaped per-expert
bias, the router's top-K choice and softmax gates, hidden rows, expert weights
and upstream gradients.  It holds none of the arithmetic of the balancing
method itself (counting, planning, destinations, permute, expert FFN,
combine, gradient reduction); that lives in ``oracle/`` (reference) and in the
HIP library (product), which never import each other.

Workload shapes follow the MoonEP pages: S tokens per EP rank, top-K routing
over E experts split into R home groups of E/R, SwiGLU experts of hidden size H
and intermediate size I (MoonEP announcement, "Technical Details"; twodots.gr
article, "memory contract"; thakicloud.com post, "What we measured", Table 2).

Conventions (fixed here so both sides read the same bytes):

* ``topk[R, S, K]`` int32, row-major in (rank, token, k).  k orders a token's
  experts by descending biased logit; equal logits go to the lower expert id.
* ``gates[R, S, K]`` float32: softmax over the K selected biased logits,
  computed in float64 then rounded once to float32.
* bf16 tensors are carried in numpy as ``uint16`` bit patterns (numpy has no
  bfloat16); conversion from float32 rounds to nearest, ties to even.
* Expert weights: ``w13[E, H, 2I]`` (gate columns ``[0, I)``, up columns
  ``[I, 2I)``) and ``w2[E, I, H]``, i.e. ``y = (silu(x W1) * (x W3)) W2``.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "bf16_bits", "bf16_to_f32", "zipf_bias", "base_logits",
    "route", "expert_load_maxvio", "tune_lambda", "routing_for", "hidden_rows", "LOGNORMAL",
    "lognormal_routing",
    "expert_weights_np", "expert_weights_torch", "grad_rows",
]


# ----------------------------------------------------------------------------
# bf16 <-> f32 bit helpers (storage format only)
# ----------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Workload configurations
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    R: int            # emulated EP ranks
    E: int            # routed experts (E/R home experts per rank)
    B: int            # prefetch slots per rank
    S: int            # tokens per rank
    K: int            # experts per token
    H: int            # hidden size
    I: int            # SwiGLU intermediate size (0: no expert GEMM in this workload)
    dtype: str        # "f32" or "bf16" hidden rows
    lam: Optional[float] = None      # explicit Zipf exponent of the router bias
    maxvio: Optional[float] = None   # target expert-level maxvio (lambda is bisected)
    seed: int = 0

    @property
    def G(self) -> int:
        return self.E // self.R

    @property
    def C(self) -> int:
        return self.S * self.K

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny CPU-checkable layer, Zipf(1.0) router bias, fp32 rows
    "tiny": Config("tiny", R=4, E=16, B=4, S=64, K=2, H=128, I=256, dtype="f32", lam=1.0),
    # plan + dispatch + combine, unbiased router
    "balanced": Config("balanced", R=8, E=256, B=4, S=4096, K=8, H=7168, I=0, dtype="bf16", lam=0.0),
    # same shapes, skewed router (maxvio set by the bias exponent)
    "skew": Config("skew", R=8, E=256, B=4, S=4096, K=8, H=7168, I=0, dtype="bf16", maxvio=4.0),
    # full expert layer forward; the inference variant uses B=3
    "layer": Config("layer", R=8, E=256, B=4, S=4096, K=8, H=7168, I=2048, dtype="bf16", maxvio=4.0),
    # training forward + backward
    "train": Config("train", R=8, E=256, B=4, S=4096, K=8, H=7168, I=2048, dtype="bf16", maxvio=4.0),
}

SKEW_SWEEP = (0.5, 2.0, 4.0, 8.0)
TRAIN_SWEEP = (0.0, 4.0, 8.0)


# ----------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------

def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def zipf_bias(E: int, lam: float) -> np.ndarray:
    """Per-expert logit bias -lam*ln(e+1): expert popularity ~ (e+1)^-lam, hottest experts first."""
    return (-float(lam) * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


@functools.lru_cache(maxsize=4)
def base_logits(R: int, S: int, E: int, seed: int) -> np.ndarray:
    """Unbiased router logits N(0,1), float32 [R*S, E], rows in (rank, token) order."""
    out = _rng(seed, 1).standard_normal((R * S, E), dtype=np.float32)
    out.setflags(write=False)
    return out


def _topk_fast(logits: np.ndarray, K: int) -> np.ndarray:
    # unordered top-K sets; only used while bisecting the bias exponent
    return np.argpartition(-logits, K - 1, axis=1)[:, :K]


def route(logits: np.ndarray, bias: np.ndarray, R: int, S: int, K: int):
    """Router top-K with softmax gates.  Returns (topk int32 [R,S,K], gates float32 [R,S,K])."""
    z = logits + bias[None, :]
    order = np.argsort(-z, axis=1, kind="stable")[:, :K]      # ties -> lower expert id
    sel = np.take_along_axis(z, order, axis=1).astype(np.float64)
    sel -= sel.max(axis=1, keepdims=True)
    ex = np.exp(sel)
    gates = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return (order.astype(np.int32).reshape(R, S, K), gates.reshape(R, S, K))


def expert_load_maxvio(topk: np.ndarray, E: int) -> float:
    """Workload knob: (max - mean)/mean of the per-expert pick counts of a routing."""
    load = np.bincount(np.asarray(topk).ravel(), minlength=E).astype(np.float64)
    return float((load.max() - load.mean()) / load.mean())


@functools.lru_cache(maxsize=32)
def tune_lambda(R: int, S: int, E: int, K: int, seed: int, target: float,
                iters: int = 40, tol: float = 0.01) -> float:
    """Bisect the Zipf exponent on [0, 4] so the routing's expert-level maxvio hits `target` (+-1%)."""
    if target <= 0.0:
        return 0.0
    logits = base_logits(R, S, E, seed)
    lo, hi = 0.0, 4.0
    lam = hi
    for _ in range(iters):
        lam = 0.5 * (lo + hi)
        mv = expert_load_maxvio(_topk_fast(logits + zipf_bias(E, lam)[None, :], K), E)
        if abs(mv - target) <= tol * target:
            break
        if mv < target:
            lo = lam
        else:
            hi = lam
    return lam


def routing_for(cfg: Config):
    """(topk, gates, lam) for a named configuration."""
    if cfg.lam is not None:
        lam = float(cfg.lam)
    else:
        lam = tune_lambda(cfg.R, cfg.S, cfg.E, cfg.K, cfg.seed, float(cfg.maxvio or 0.0))
    topk, gates = route(base_logits(cfg.R, cfg.S, cfg.E, cfg.seed), zipf_bias(cfg.E, lam),
                        cfg.R, cfg.S, cfg.K)
    return topk, gates, lam


# Lognormal expert popularity (the planner workload of the thakicloud.com post, "What we
# measured", Table 1: 256 experts, 8 ranks, 2048 tokens per rank, top-8, skew set by a
# lognormal sigma).  The post's generator is not available; this one samples each token's K
# experts without replacement with probabilities proportional to w_e = exp(sigma * z_e),
# z_e ~ N(0, 1) (Gumbel top-K: argsort of log w_e + Gumbel noise).  sigma = 0 is uniform
# random routing, not the exactly balanced assignment the post's generator makes.
LOGNORMAL = dict(R=8, E=256, S=2048, K=8, sigmas=(0.0, 0.5, 1.0, 2.0, 5.0))


@functools.lru_cache(maxsize=8)
def lognormal_routing(R: int, S: int, E: int, K: int, sigma: float, seed: int = 0):
    """(topk int32 [R,S,K], gates float32 [R,S,K]); ties to the lower expert id."""
    logw = (float(sigma) * _rng(seed, 5).standard_normal(E)).astype(np.float64)
    u = _rng(seed, 6).random((R * S, E))
    gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0 - 1e-16)))
    z = logw[None, :] + gumbel
    order = np.argsort(-z, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(z, order, axis=1)
    sel -= sel.max(axis=1, keepdims=True)
    ex = np.exp(sel)
    gates = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    topk = order.astype(np.int32).reshape(R, S, K)
    topk.setflags(write=False)
    return topk, gates.reshape(R, S, K)


# ----------------------------------------------------------------------------
# Hidden rows, weights, upstream gradients
# ----------------------------------------------------------------------------

def hidden_rows(R: int, S: int, H: int, seed: int, dtype: str) -> np.ndarray:
    """x ~ N(0,1) [R,S,H]: float32 for dtype 'f32', bf16 bits (uint16) for 'bf16'."""
    x = _rng(seed, 2).standard_normal((R, S, H), dtype=np.float32)
    return x if dtype == "f32" else bf16_bits(x)


def grad_rows(R: int, S: int, H: int, seed: int, dtype: str) -> np.ndarray:
    """Upstream gradient dOut ~ N(0,1) [R,S,H] (same storage rules as hidden_rows)."""
    g = _rng(seed, 3).standard_normal((R, S, H), dtype=np.float32)
    return g if dtype == "f32" else bf16_bits(g)


def expert_weights_np(E: int, H: int, I: int, seed: int, std: float = 0.02):
    """(w13 [E,H,2I], w2 [E,I,H]) ~ N(0, std^2) as float32 (small configurations)."""
    rng = _rng(seed, 4)
    w13 = (rng.standard_normal((E, H, 2 * I), dtype=np.float32) * np.float32(std))
    w2 = (rng.standard_normal((E, I, H), dtype=np.float32) * np.float32(std))
    return w13, w2


def expert_weights_torch(E: int, H: int, I: int, seed: int, device, std: float = 0.02):
    """(w13 [E,H,2I], w2 [E,I,H]) ~ N(0, std^2) in bf16, drawn by torch's generator on `device`.

    Used where the weights are too large to draw on the host (tens of GB).  Draws one
    expert at a time in float32 and rounds to bf16 (round to nearest even).
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 4)
    w13 = torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w13[e].copy_(torch.randn((H, 2 * I), generator=gen, device=device, dtype=torch.float32) * std)
        w2[e].copy_(torch.randn((I, H), generator=gen, device=device, dtype=torch.float32) * std)
    return w13, w2
