"""Oracle: router projection, scores, top-k selection and gates (float64).

Test infrastructure only (see ``oracle/__init__.py``).

Follows
* [Switch review] "Switch Routing 메커니즘": Step 1 h(x) = x·W_r, p_i = e^{h_i}/Σ_j e^{h_j};
  Step 2 i* = argmax_i p_i; Step 3 y = p_{i*}(x)·E_{i*}(x) (the gate is the
  router probability of the chosen expert).
* [Switch review] "선택적 정밀도 캐스팅": bf16 hidden states are upcast (exactly)
  and the router runs in high precision.  The oracle runs it in float64.
* [Switch review] "Shazeer et al. (2017)의 MoE Layer": top-k gating
  g = Softmax(TopK(x·W_g)) — the renormalised top-k gate (``gate="renorm"``).
* [MoE tour 6] "방법 회고" eq. (1): Loss-Free routing picks argtop-k of ρ + b but
  weights the expert by ρ_i alone; ρ = sigmoid(h) in that setting.

Readings (pages silent): ranking without a bias uses the logits h, which is
the same order as p or sigmoid(h) because both are strictly increasing in h.
Ties go to the lower expert index; the k choices of a token are listed by
descending key.  With a bias the key is score + bias, score = p or sigmoid(h).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def decode_hidden(x) -> np.ndarray:
    """Exact float64 value of the stored hidden states (uint16 = bf16 bit patterns)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def logits(x, w_r) -> np.ndarray:
    """h = x · W_r in float64; W_r is [d, n] ([Switch review] Step 1)."""
    return decode_hidden(x) @ np.asarray(w_r, dtype=np.float64)


def softmax(h: np.ndarray) -> np.ndarray:
    """p_i = e^{h_i} / Σ_j e^{h_j} per row ([Switch review] Step 1)."""
    e = np.exp(h - h.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def sigmoid(h: np.ndarray) -> np.ndarray:
    """ρ = 1 / (1 + e^{-h}) ([MoE tour 6] "방법 회고": sigmoid-activated scores)."""
    return 1.0 / (1.0 + np.exp(-h))


def scores(h: np.ndarray, score: str) -> np.ndarray:
    if score == "softmax":
        return softmax(h)
    if score == "sigmoid":
        return sigmoid(h)
    raise ValueError(score)


def ranking_keys(h: np.ndarray, score: str, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Key whose top-k is the selection: h without a bias, score + b with one (eq. (1))."""
    if bias is None:
        return h
    return scores(h, score) + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]


def topk(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, by descending key, lower index first on ties."""
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def near_tie_margin(keys: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap among the sorted top-(k+1) keys, relative to the row's largest |key|.

    A token whose margin is below 1e-6 has a selection that rounding of the
    keys can change; such tokens are reported apart from the exact-match check.
    With k == n only the gaps inside the top k count.
    """
    srt = -np.sort(-keys, axis=1)
    n = keys.shape[1]
    upto = min(k + 1, n)
    gaps = srt[:, : upto - 1] - srt[:, 1:upto]
    if gaps.shape[1] == 0:
        return np.full(keys.shape[0], np.inf)
    scale = np.maximum(np.abs(keys).max(axis=1), np.finfo(np.float64).tiny)
    return gaps.min(axis=1) / scale


def gates(h: np.ndarray, idx: np.ndarray, score: str, gate: str = "prob") -> np.ndarray:
    """Gate per (token, choice): the chosen expert's score ([Switch review] Step 3,
    [MoE tour 6] eq. (1)); ``renorm`` divides by the sum over the k choices
    (Softmax over TopK for softmax scores)."""
    s = scores(h, score)
    g = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    if gate == "renorm":
        g = g / g.sum(axis=1, keepdims=True)
    elif gate != "prob":
        raise ValueError(gate)
    return g


@dataclass
class Route:
    idx: np.ndarray        # [m, k] int32
    gate: np.ndarray       # [m, k] float64
    probs: np.ndarray      # [m, n] float64 (p or sigmoid scores)
    keys: np.ndarray       # [m, n] float64
    margin: np.ndarray     # [m]
    counts: np.ndarray     # [n] int64 (selections before any capacity limit)
    prob_sum: np.ndarray   # [n] Σ_t p_j(t)

    def near_ties(self, rel: float = 1e-6) -> np.ndarray:
        return np.nonzero(self.margin < rel)[0]


def route(x, w_r, k: int, score: str = "softmax", bias=None, gate: str = "prob") -> Route:
    h = logits(x, w_r)
    p = scores(h, score)
    keys = ranking_keys(h, score, bias)
    idx = topk(keys, k)
    g = gates(h, idx, score, gate)
    n = h.shape[1]
    counts = np.bincount(idx.reshape(-1), minlength=n).astype(np.int64)
    return Route(idx, g, p, keys, near_tie_margin(keys, k), counts, p.sum(axis=0))
