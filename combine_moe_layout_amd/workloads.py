"""Seeded synthetic inputs for MoE dispatch / combine.

This module only draws inputs: token hidden states, router top-k choices and
routing weights, and (for combine-only checks) random expert outputs.  It holds
none of the dispatch / combine arithmetic, so the oracle and the HIP path can
both be fed from it.

Workloads follow the pages' benchmark dimensions (tokens per rank, top-k,
hidden, precision, uniform vs skewed routing: "DeepEP是什麼？…" (yololab.net),
section "Benchmark矩陣") and the DeepSeek-V3-style test configuration of 8K
tokens, hidden 7168, FP8 dispatch and BF16 combine (DeepEP v2 release notes,
donniechu.com, section "Số liệu kỹ thuật") with 256 experts and top-8
("DeepEP 编址服务深度对抗分析", section 五.2).  Router top-k itself is
upstream of the path; here it is only a generator.

Random streams: numpy ``default_rng([seed, stream])``; stream 0 draws x,
stream 1 draws the routing, stream 2 draws random expert outputs.  x is
float32 N(0,1) rounded to bf16 (nearest-even) and kept as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses

import numpy as np

STREAM_X, STREAM_ROUTING, STREAM_Y = 0, 1, 2


@dataclasses.dataclass
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden
    E: int            # experts
    G: int            # logical groups (stand-ins for EP ranks)
    k: int            # top-k
    cap: int          # 0: contiguous receive layout; >0: padded, cap rows per expert
    fp8: bool         # FP8 e4m3 dispatch (else bf16)
    x_bits: np.ndarray        # uint16 [T, H], bf16 bit patterns
    topk_idx: np.ndarray      # int64  [T, k]
    topk_weights: np.ndarray  # float32 [T, k]

    @property
    def R(self) -> int:
        """Receive rows: T*k contiguous, or E*cap padded."""
        return self.E * self.cap if self.cap > 0 else self.T * self.k


def float32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); inputs here are finite."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def draw_x(T: int, H: int, seed: int = 0) -> np.ndarray:
    g = _rng(seed, STREAM_X)
    return float32_to_bf16_bits(g.standard_normal((T, H), dtype=np.float32))


def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, largest first, ties to the lower id."""
    return np.argsort(-scores, axis=1, kind="stable")[:, :k].astype(np.int64)


def _softmax_selected(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
    sel = sel - sel.max(axis=1, keepdims=True)
    e = np.exp(sel)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def route_uniform(T: int, E: int, k: int, seed: int = 0, normal: bool = False):
    """top-k of i.i.d. logits (U(0,1), or N(0,1) if normal); weights = softmax
    over the k selected logits."""
    g = _rng(seed, STREAM_ROUTING)
    logits = g.standard_normal((T, E)) if normal else g.random((T, E))
    idx = _topk_desc(logits, k)
    return idx, _softmax_selected(logits, idx)


def route_skewed(T: int, E: int, k: int, G: int, groups_kept: int, s: float = 1.2, seed: int = 0):
    """Zipf(s) expert popularity p_e ~ (e+1)^-s; scores log p + Gumbel(0,1)
    (Gumbel-top-k = sampling without replacement in proportion to p); a
    group's score is its best member's; keep the best `groups_kept` groups,
    then the top-k experts inside them; weights = softmax of the kept scores."""
    g = _rng(seed, STREAM_ROUTING)
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    scores = np.log(p)[None, :] + g.gumbel(size=(T, E))
    per = E // G
    gscore = scores.reshape(T, G, per).max(axis=2)
    keep = _topk_desc(gscore, groups_kept)                   # [T, groups_kept]
    mask = np.zeros((T, G), bool)
    np.put_along_axis(mask, keep, True, axis=1)
    masked = np.where(np.repeat(mask, per, axis=1), scores, -np.inf)
    idx = _topk_desc(masked, k)
    return idx, _softmax_selected(scores, idx)


def route_shared(T: int, E: int, k: int, seed: int = 0):
    """Expert 0 is a shared expert, always at position j = 0; the other k-1 are
    the top of N(0,1) logits over experts 1..E-1; weights = softmax over the k
    selected logits (the shared expert's logit is drawn like the rest)."""
    g = _rng(seed, STREAM_ROUTING)
    logits = g.standard_normal((T, E))
    routed = _topk_desc(logits[:, 1:], k - 1) + 1
    idx = np.concatenate([np.zeros((T, 1), np.int64), routed], axis=1)
    return idx, _softmax_selected(logits, idx)


def random_expert_outputs(R: int, H: int, seed: int = 0) -> np.ndarray:
    """Random bf16 expert outputs, N(0,1), for combine-only checks."""
    g = _rng(seed, STREAM_Y)
    return float32_to_bf16_bits(g.standard_normal((R, H), dtype=np.float32))


# name -> (T, H, E, G, k, cap, fp8, routing)
CONFIGS = {
    "tiny":    (128, 256, 8, 1, 2, 0, False, "softmax_normal"),
    "dsv3":    (8192, 7168, 256, 8, 8, 0, True, "uniform"),
    "skewed":  (8192, 7168, 256, 8, 8, 0, False, "skewed"),
    "lowlat":  (128, 7168, 256, 8, 8, 128, True, "uniform"),
    "large":   (65536, 4096, 64, 8, 6, 0, True, "shared"),
}

DESCRIPTIONS = {
    "tiny": "T=128 H=256 E=8 top-2 bf16 dispatch/combine",
    "dsv3": "DeepSeek-V3-style prefill: T=8192 H=7168 E=256 (8 groups of 32) top-8, "
            "FP8 e4m3 dispatch (fp32 scale per 128 ch), bf16 combine",
    "skewed": "T=8192 H=7168 E=256 top-8, Zipf(1.2) popularity, top-4-of-8 groups, bf16",
    "lowlat": "T=128 H=7168 E=256 top-8, FP8 dispatch into padded buffer (cap 128/expert)",
    "large": "T=65536 H=4096 E=64 top-6 incl. shared expert 0, FP8 dispatch, bf16 combine",
}


def route(kind: str, T: int, E: int, k: int, G: int, seed: int = 0):
    if kind == "uniform":
        return route_uniform(T, E, k, seed)
    if kind == "softmax_normal":
        return route_uniform(T, E, k, seed, normal=True)
    if kind == "skewed":
        return route_skewed(T, E, k, G, groups_kept=min(4, G), seed=seed)
    if kind == "shared":
        return route_shared(T, E, k, seed)
    raise ValueError("unknown routing kind %r" % kind)


def make(name: str, seed: int = 0, T: int | None = None, H: int | None = None) -> Workload:
    """One of the named workloads, optionally with fewer tokens or a smaller
    hidden size (same routing recipe) for checks the oracle finishes quickly."""
    T0, H0, E, G, k, cap, fp8, kind = CONFIGS[name]
    T = T0 if T is None else T
    H = H0 if H is None else H
    idx, w = route(kind, T, E, k, G, seed)
    return Workload(name, T, H, E, G, k, cap, fp8, draw_x(T, H, seed), idx, w)


def custom(T: int, H: int, E: int, k: int, G: int = 1, cap: int = 0, fp8: bool = False,
           routing: str = "uniform", seed: int = 0) -> Workload:
    idx, w = route(routing, T, E, k, G, seed) if T > 0 else (
        np.zeros((0, k), np.int64), np.zeros((0, k), np.float32))
    return Workload("custom", T, H, E, G, k, cap, fp8, draw_x(T, H, seed), idx, w)
