"""Oracle: expert FFN (ReLU, bf16 weights) and gate-scaled combine with residual.

Test infrastructure only (see ``oracle/__init__.py``).

Follows
* [Switch review] "Switch Layer의 구조": FFN(x) = max(0, x·W1 + b1)·W2 + b2,
  replicated as N experts with their own weights.  The workloads carry no
  biases, so b1 = b2 = 0 (a reading).
* [Switch review] "Switch Routing 메커니즘" Step 3 and the Shazeer sum
  y = Σ_i g_i(x)·E_i(x): the layer output scales each expert output by its gate.
* [Switch impl] "Switch Transformer를 구현 관점에서 읽기" (pipeline list) and
  "Expert Capacity를 구체적으로 계산한다": the gated expert output joins the
  residual path; dropped (overflow) tokens only take the residual path.

Precision (reading of [Switch impl] "Router만 float32로 올리는 Selective
Precision": only the router is fp32, the experts run in bf16): products are
formed exactly in float64, the hidden activation is rounded to bf16 (nearest
even) and so is the expert output.  The combine is computed in float64 and
rounded to the storage dtype of x.
"""
from __future__ import annotations

import numpy as np


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    Finite values inside the fp32 normal range; works on the float64 bit
    pattern: bf16 keeps 7 fraction bits, float64 has 52, so the rounding
    position is fraction bit 45.
    """
    u = np.ascontiguousarray(v, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of float64 values."""
    r = bf16_round(v).astype(np.float32)        # exact: r is bf16-representable
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def relu_ffn(rows64: np.ndarray, w1_bits: np.ndarray, w2_bits: np.ndarray) -> np.ndarray:
    """Y = bf16(bf16(max(0, D·W1)) · W2) for one expert, as float64.

    w1_bits: [d_ff, d] (math W1 = w1^T); w2_bits: [d, d_ff] (math W2 = w2^T).
    """
    W1 = from_bf16_bits(w1_bits).T
    W2 = from_bf16_bits(w2_bits).T
    H = bf16_round(np.maximum(rows64 @ W1, 0.0))
    return bf16_round(H @ W2)


def combine(x64: np.ndarray, y64: np.ndarray, gate: np.ndarray, token_to_row: np.ndarray,
            residual: bool = True) -> np.ndarray:
    """out[t] = x[t] + Σ_{r kept} gate[t,r] · y[row(t,r)]  (float64, unrounded)."""
    T, k = token_to_row.shape
    out = x64.copy() if residual else np.zeros_like(x64)
    for r in range(k):
        rows = token_to_row[:, r]
        keep = rows >= 0
        out[keep] += np.asarray(gate, np.float64)[keep, r][:, None] * y64[rows[keep]]
    return out
