"""Oracle: load statistics, Switch aux loss, global-batch accumulation, Loss-Free bias.

Test infrastructure only (see ``oracle/__init__.py``).

Follows
* [Switch review] "로드 밸런싱 손실": L_aux = α·N·Σ_i f_i·P_i with
  f_i = (1/T) Σ_x 1{argmax p(x) = i} and P_i = (1/T) Σ_x p_i(x); balanced routing
  (f_i = P_i = 1/N) gives L_aux = α.  For k > 1 the oracle keeps f_i = c_i / T,
  the fraction of tokens that selected expert i (a reading; the page is top-1).
* [Qwen global] "글로벌-배치 로드 밸런스 구현": f_i is gathered over the whole
  global batch (all micro-batches), the loss is then formed per micro-batch
  with that global f, and the per-micro-batch losses are averaged.  The same
  page's hybrid ("효율성과 효과성의 균형"): the micro-batch balance loss
  (the Switch loss of each micro-batch on its own f) is added to the global
  one with a constant weight 0.01.  The page's parenthetical attaches that
  weight to the global-batch loss; the sentence it sits in adds the
  micro-batch loss.  Both readings are kept by taking two weights:
  L_hybrid^(t) = w_g · L_global^(t) + w_m · L_micro^(t), averaged like the
  global one; reading A (micro-batch loss weighted) is (w_g, w_m) = (1, 0.01),
  reading B (global loss weighted) is (0.01, 1).
* [MoE tour 6] "방법 회고" eq. (2): b ← b − γ·sign(F − 1/n), F = observed load
  share; applied after routing with the old b ("함정에 주의").  The bias is fp32
  state, so this update is computed in fp32: F_j − 1/n has the sign of
  c_j·n − m·k, evaluated exactly in integers, and b_j − fl32(γ)·s_j is one fp32
  operation.
* [MoE tour 6] "방법 회고" and "데모 코드": the load share F_j = c_j / Σ c
  against its expected value 1/n; the violation of expert j is the relative
  excess F_j / (1/n) − 1, and the page reports its maximum (MaxVio, ≥ 0), its
  minimum (≥ −1) and its mean absolute value, all 0 when perfectly balanced.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np


def counts(idx: np.ndarray, n: int) -> np.ndarray:
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n).astype(np.int64)


def switch_stats(c: np.ndarray, prob_sum: np.ndarray, m: int, alpha: float):
    """(f, P, aux) in float64 for a batch of m tokens."""
    c = np.asarray(c, dtype=np.float64)
    n = c.shape[0]
    f = c / m
    P = np.asarray(prob_sum, dtype=np.float64) / m
    aux = alpha * n * float(np.sum(f * P))
    return f, P, aux


@dataclass
class GlobalBatch:
    """Accumulates expert counts over micro-batches ([Qwen global])."""
    n: int
    counts: np.ndarray = None
    tokens: int = 0
    prob_means: List[np.ndarray] = field(default_factory=list)

    def __post_init__(self):
        if self.counts is None:
            self.counts = np.zeros(self.n, dtype=np.int64)

    micro_f: List[np.ndarray] = field(default_factory=list)

    def add(self, c: np.ndarray, m: int, prob_sum: np.ndarray = None):
        self.counts = self.counts + np.asarray(c, dtype=np.int64)
        self.tokens += int(m)
        if prob_sum is not None:
            self.prob_means.append(np.asarray(prob_sum, dtype=np.float64) / m)
            self.micro_f.append(np.asarray(c, dtype=np.float64) / m)

    def f(self) -> np.ndarray:
        return self.counts.astype(np.float64) / self.tokens

    def losses(self, alpha: float) -> np.ndarray:
        """L^(t) = α·N·Σ_i f_i^global · P_i^(t) for each micro-batch t."""
        fg = self.f()
        return np.array([alpha * self.n * float(np.sum(fg * P)) for P in self.prob_means])

    def loss(self, alpha: float) -> float:
        return float(np.mean(self.losses(alpha)))

    def micro_losses(self, alpha: float) -> np.ndarray:
        """The Switch loss of each micro-batch with its own f: α·N·Σ_i f_i^(t) · P_i^(t)."""
        return np.array([alpha * self.n * float(np.sum(f * P)) for f, P in zip(self.micro_f, self.prob_means)])

    def hybrid_losses(self, alpha: float, w_global: float, w_micro: float) -> np.ndarray:
        """w_global · L_global^(t) + w_micro · L_micro^(t) for each micro-batch t."""
        return w_global * self.losses(alpha) + w_micro * self.micro_losses(alpha)

    def hybrid_loss(self, alpha: float, w_global: float, w_micro: float) -> float:
        return float(np.mean(self.hybrid_losses(alpha, w_global, w_micro)))


def lossfree_update(bias: np.ndarray, c: np.ndarray, m: int, k: int, gamma: float) -> np.ndarray:
    """One Loss-Free step in fp32: b_j ← b_j − fl32(γ)·sign(c_j·n − m·k)."""
    b = np.asarray(bias, dtype=np.float32)
    n = b.shape[0]
    s = np.sign(np.asarray(c, dtype=np.int64) * n - np.int64(m) * k).astype(np.float32)
    return (b - np.float32(gamma) * s).astype(np.float32)


def load_violation(c: np.ndarray):
    """(MaxVio, min, mean |·|) of each expert's relative excess load F_j·n − 1, where
    F_j = c_j / Σ c is its load share and 1/n the balanced share."""
    c = np.asarray(c, dtype=np.float64)
    n = c.shape[0]
    share = c / c.sum()
    excess = share / (1.0 / n) - 1.0
    return float(excess.max()), float(excess.min()), float(np.mean(np.abs(excess)))
