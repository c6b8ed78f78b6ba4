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
given in token-major order (token t before t+1, then choice r before r+1).
Two buffer layouts, both expert-major: compact (expert j's kept rows follow
expert j-1's, offsets are prefix sums of the kept counts — the grouping the
permute example on [Switch impl] draws), and capacity-padded (expert j owns
rows [j·C, (j+1)·C) and fills the first kept_j of them — the per-expert
capacity buffer of [Switch review] "Expert Capacity와 토큰 드롭").  Slots,
kept / dropped pairs and the row order inside an expert are the same in both.
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
    kept_counts: np.ndarray     # [n] min(counts, capacity) = rows filled per expert
    padded: bool = False        # capacity-padded layout (expert j owns rows [j·C, (j+1)·C))

    @property
    def rows(self) -> int:
        """Rows of the dispatched buffer (padded: n·C, some of them unfilled)."""
        return int(self.expert_offsets[-1])

    @property
    def expert_rows(self) -> np.ndarray:
        """[n] int32: filled rows of each expert, from its offset on."""
        return self.kept_counts.astype(np.int32)

    def filled_rows(self) -> np.ndarray:
        """Indices of the dispatched rows that hold a token."""
        return np.nonzero(self.row_to_token >= 0)[0]


def dispatch_maps(idx: np.ndarray, n: int, cap: int, padded: bool = False) -> Dispatch:
    """Slots in token order and the permute maps; padded needs cap >= 0."""
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
    if padded:
        assert cap >= 0, "the padded layout needs a capacity"
        offsets[:] = np.arange(n + 1) * cap
    else:
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
                    counts, kept_counts, padded)


def dispatch_rows(x: np.ndarray, dm: Dispatch) -> np.ndarray:
    """Dispatched buffer: row r holds the (bit-identical) hidden state of its
    token; unfilled rows of the padded layout are zero."""
    x = np.asarray(x)
    out = np.zeros((dm.rows,) + x.shape[1:], dtype=x.dtype)
    filled = dm.filled_rows()
    out[filled] = x[dm.row_to_token[filled]]
    return out
