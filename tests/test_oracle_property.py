"""Property tests of the oracle (hypothesis, derandomised; CPU): random small routings with
integer-valued x and W_r (exact logits, so ties are real) against brute force written
independently of the oracle's code:
  - top-k: Python's sorted() over (-key, expert), so ties go to the lower expert
    ([Switch review] "Switch Routing 메커니즘": the argmax, generalised to k picks);
  - slots: a direct count of earlier (token, choice) pairs on the same expert in token-major
    order, kept iff below the capacity ([Switch review] "Expert Capacity와 토큰 드롭");
  - maps: token_to_row and row_to_token are inverse on the kept pairs, each expert's rows are
    contiguous from its offset, kept = min(count, C) and the drops add up."""
import numpy as np
import pytest

from oracle import dispatch as OD
from oracle import router as OR

hyp = pytest.importorskip("hypothesis")
st = hyp.strategies


@hyp.settings(max_examples=80, deadline=None, derandomize=True, database=None,
              suppress_health_check=list(hyp.HealthCheck))
@hyp.given(m=st.integers(1, 60), n=st.integers(1, 12), k=st.integers(1, 4), d=st.integers(1, 6),
           cf=st.sampled_from([-1.0, 0.0, 0.5, 1.0, 2.0]), score=st.sampled_from(["softmax", "sigmoid"]),
           padded=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_route_and_dispatch_against_brute_force(m, n, k, d, cf, score, padded, seed):
    k = min(k, n)
    rng = np.random.default_rng(seed)
    x = rng.integers(-2, 3, (m, d)).astype(np.float32)
    w = rng.integers(-1, 2, (d, n)).astype(np.float32)
    r = OR.route(x, w, k, score=score)
    h = x.astype(np.int64) @ w.astype(np.int64)            # exact integer logits
    for t in range(m):
        want = sorted(range(n), key=lambda j: (-int(h[t, j]), j))[:k]
        assert [int(v) for v in r.idx[t]] == want
    assert np.array_equal(r.counts, np.bincount(r.idx.ravel(), minlength=n))
    cap = int(cf * m * k / n) if cf >= 0 else m * k
    padded = padded and cf >= 0
    dm = OD.dispatch_maps(r.idx, n, cap, padded=padded)
    seen = [0] * n
    kept = np.zeros((m, k), bool)
    for t in range(m):
        for c in range(k):
            e = int(r.idx[t, c])
            kept[t, c] = seen[e] < cap
            seen[e] += 1
    assert np.array_equal(dm.drop_mask == 0, kept)
    kept_counts = np.minimum(r.counts, cap)
    assert int((~kept).sum()) == int(np.maximum(r.counts - cap, 0).sum())
    for e in range(n):
        base = e * cap if padded else int(kept_counts[:e].sum())
        assert dm.expert_offsets[e] == base
        rows = sorted(int(dm.token_to_row[t, c]) for t in range(m) for c in range(k)
                      if kept[t, c] and r.idx[t, c] == e)
        assert rows == list(range(base, base + int(kept_counts[e])))
    for t in range(m):
        for c in range(k):
            row = int(dm.token_to_row[t, c])
            assert (row >= 0) == kept[t, c]
            if row >= 0:
                assert dm.row_to_token[row] == t
