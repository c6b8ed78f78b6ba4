"""Oracle: expert capacity, slots in token order, permute-dispatch maps.

Test infrastructure only (see ``oracle/__init__.py``).

Follows
* [Switch review] "Expert Capacity와 토큰 드롭": capacity = (tokens per batch /
  number of experts) × capacity factor; tokens beyond it skip the expert and
  reach the next layer through the residual connection.
* [Switch impl] "Expert Capacity를 구체적으로 계산한다": overflow tokens pass
  through the residual path (they stay in the sequence).
* [Switch impl] "forward pass에서는 토큰 순서를 두 번 변경한다": tokens that chose
  the same expert are gathered together (permute), the expert runs batched,
  the original order is restored (inverse permute); each token keeps its gate
  and capacity slot.

Readings: capacity = floor(T·cf / N) on the exact value of cf; slots are
given in token-major order (token t before t+1, then choice r before r+1);
the dispatched buffer is compact and expert-major with row offsets.
Plain Python loops: fine at the sizes the oracle runs.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np


def capacity(T: int, n: int, cf: float) -> int:
    """floor(T · cf / n) in exact rational arithmetic."""
    return int(Fraction(T) * Fraction(cf) / Fraction(n)) if cf >= 0 else -1


@dataclass
class Dispatch:
    slot: np.ndarray            # [T, k] int64: rank among earlier pairs of the same expert
    kept: np.ndarray            # [T, k] bool
    token_to_row: np.ndarray    # [T, k] int32, -1 if dropped
    drop_mask: np.ndarray       # [T, k] uint8, 1 if dropped
    expert_offsets: np.ndarray  # [n + 1] int32
    row_to_token: np.ndarray    # [rows] int32 (token index of each dispatched row)
    row_to_pair: np.ndarray     # [rows] int64 (flat t*k + r of each row)
    counts: np.ndarray          # [n] selections
    kept_counts: np.ndarray     # [n] min(counts, capacity)

    @property
    def rows(self) -> int:
        return int(self.expert_offsets[-1])


def dispatch_maps(idx: np.ndarray, n: int, cap: int) -> Dispatch:
    idx = np.asarray(idx)
    T, k = idx.shape
    slot = np.zeros((T, k), dtype=np.int64)
    cnt = [0] * n
    for t in range(T):                     # token order ...
        for r in range(k):                 # ... then choice order
            e = int(idx[t, r])
            slot[t, r] = cnt[e]
            cnt[e] += 1
    counts = np.array(cnt, dtype=np.int64)
    kept = slot < cap
    kept_counts = np.minimum(counts, cap)
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_counts)
    token_to_row = np.full((T, k), -1, dtype=np.int64)
    rows = int(offsets[-1])
    row_to_token = np.full(rows, -1, dtype=np.int64)
    row_to_pair = np.full(rows, -1, dtype=np.int64)
    for t in range(T):
        for r in range(k):
            if kept[t, r]:
                row = offsets[idx[t, r]] + slot[t, r]
                token_to_row[t, r] = row
                row_to_token[row] = t
                row_to_pair[row] = t * k + r
    return Dispatch(slot, kept, token_to_row.astype(np.int32), (~kept).astype(np.uint8),
                    offsets.astype(np.int32), row_to_token.astype(np.int32), row_to_pair,
                    counts, kept_counts)


def dispatch_rows(x: np.ndarray, dm: Dispatch) -> np.ndarray:
    """Dispatched buffer: row r holds the (bit-identical) hidden state of its token."""
    return np.asarray(x)[dm.row_to_token]
