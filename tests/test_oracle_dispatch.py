"""Pins of the capacity / slot / dispatch oracle and the expert + combine oracle (CPU only)."""
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dispatch as D
from oracle import expert as E

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.setdefault(parts[0], []).append(parts[1:])
    return rows


def test_permute_worked_example():
    g = _read_golden("permute_example.txt")
    experts = np.array([int(v) - 1 for v in g["experts"][0]], np.int32)[:, None]
    dm = D.dispatch_maps(experts, 4, cap=6)
    assert (dm.row_to_token + 1).tolist() == [int(v) for v in g["dispatched_tokens"][0]]
    assert dm.expert_offsets.tolist() == [int(v) for v in g["expert_offsets"][0]]
    # inverse permute restores the original order
    order = np.empty(6, np.int64)
    order[dm.row_to_token] = np.arange(6)
    assert np.array_equal(dm.token_to_row[:, 0], order)


def test_permute_worked_example_row_contents():
    """dispatch_rows on the same example, against the hand-written buffers: compact, and
    capacity-padded with capacity 2 (unfilled rows zero)."""
    g = _read_golden("permute_example.txt")
    experts = np.array([int(v) - 1 for v in g["experts"][0]], np.int32)[:, None]
    x = np.array([[t, 10 * t] for t in range(1, 7)], np.float32)
    compact = np.array([[float(v) for v in r] for r in g["dispatched_row"]], np.float32)
    padded = np.array([[float(v) for v in r] for r in g["padded_row"]], np.float32)
    dm = D.dispatch_maps(experts, 4, cap=6)
    assert np.array_equal(D.dispatch_rows(x, dm), compact)
    dp = D.dispatch_maps(experts, 4, cap=2, padded=True)
    assert np.array_equal(D.dispatch_rows(x, dp), padded)
    # inverse permute of the compact buffer restores x
    assert np.array_equal(D.dispatch_rows(x, dm)[dm.token_to_row[:, 0]], x)


def _capacity_example_idx(counts, seed):
    T = sum(counts)
    idx = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    return np.random.default_rng(seed).permutation(idx).astype(np.int32)[:, None]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_capacity_worked_example(seed):
    g = _read_golden("capacity_example.txt")
    T = int(g["tokens"][0][0])
    n = int(g["experts"][0][0])
    counts = [int(v) for v in g["counts"][0]]
    idx = _capacity_example_idx(counts, seed)
    for row in g["cf"]:
        cf, cap = float(row[0]), int(row[2])
        kept = [int(v) for v in row[4:8]]
        dropped = int(row[9])
        assert D.capacity(T, n, cf) == cap
        dm = D.dispatch_maps(idx, n, cap)
        assert dm.kept_counts.tolist() == kept
        assert int(dm.drop_mask.sum()) == dropped
        # the dropped tokens of expert 0 are its last ones in token order
        t0 = np.nonzero(idx[:, 0] == 0)[0]
        assert np.all(dm.drop_mask[t0[:cap], 0] == 0)
        assert np.all(dm.drop_mask[t0[cap:], 0] == 1)


def test_capacity_is_exact_rational_floor():
    assert D.capacity(1024, 8, 1.25) == 160
    assert D.capacity(8192, 128, 1.0) == 64
    assert D.capacity(8192, 128, 1.25) == 80
    assert D.capacity(65536, 2048, 1.25) == 40
    # 0.3 is stored just below 3/10, so 10 * 0.3 / 1 is just below 3
    assert D.capacity(10, 1, 0.3) == 2
    assert D.capacity(7, 2, 0.0) == 0


@pytest.mark.parametrize("k,skew,cf", [(1, 0.0, 1.0), (1, 1.2, 1.25), (2, 0.5, 1.0), (4, 2.0, 0.5)])
def test_dispatch_invariants(k, skew, cf):
    T, n = 500, 16
    idx = W.random_assignment(T, n, k, seed=7, skew=skew)
    cap = D.capacity(T * k, n, cf)
    dm = D.dispatch_maps(idx, n, cap)
    assert dm.counts.sum() == T * k
    assert np.array_equal(dm.kept_counts, np.minimum(dm.counts, cap))
    assert dm.rows == dm.kept_counts.sum() == (dm.drop_mask == 0).sum()
    # row maps are mutually inverse
    t, r = np.nonzero(dm.token_to_row >= 0)
    assert np.array_equal(dm.row_to_token[dm.token_to_row[t, r]], t)
    # rows of expert e are its kept pairs in (token, choice) order, slots 0..kept-1
    for e in range(n):
        lo, hi = dm.expert_offsets[e], dm.expert_offsets[e + 1]
        pairs = dm.row_to_pair[lo:hi]
        assert np.all(np.diff(pairs) > 0)
        assert np.all(idx.reshape(-1)[pairs] == e)
        assert np.array_equal(dm.slot.reshape(-1)[pairs], np.arange(hi - lo))


def test_all_tokens_to_one_expert_drops_T_minus_C():
    T, n = 64, 4
    idx = np.zeros((T, 1), np.int32)
    cap = D.capacity(T, n, 1.25)
    dm = D.dispatch_maps(idx, n, cap)
    assert int(dm.drop_mask.sum()) == T - cap
    assert dm.expert_offsets.tolist() == [0, cap, cap, cap, cap]


def test_padded_permute_worked_example():
    # the permute example, each expert's group placed at the start of its capacity region
    g = _read_golden("permute_example.txt")
    experts = np.array([int(v) - 1 for v in g["experts"][0]], np.int32)[:, None]
    cap = 6
    dm = D.dispatch_maps(experts, 4, cap, padded=True)
    compact = [int(v) for v in g["dispatched_tokens"][0]]
    off = [int(v) for v in g["expert_offsets"][0]]
    assert dm.expert_offsets.tolist() == [e * cap for e in range(5)]
    for e in range(4):
        group = compact[off[e]:off[e + 1]]
        region = (dm.row_to_token[e * cap:(e + 1) * cap] + 1).tolist()
        assert region == group + [0] * (cap - len(group))
        assert dm.expert_rows[e] == len(group)


@pytest.mark.parametrize("k,skew,cf", [(1, 0.0, 1.0), (1, 1.2, 1.25), (2, 0.5, 1.0), (4, 2.0, 0.5), (2, 1.0, 0.0)])
def test_padded_layout_matches_compact(k, skew, cf):
    T, n = 400, 16
    idx = W.random_assignment(T, n, k, seed=11, skew=skew)
    cap = D.capacity(T * k, n, cf)
    c = D.dispatch_maps(idx, n, cap)
    p = D.dispatch_maps(idx, n, cap, padded=True)
    for a in ("slot", "kept", "drop_mask", "counts", "kept_counts"):
        assert np.array_equal(getattr(c, a), getattr(p, a)), a
    assert p.rows == n * cap and len(p.filled_rows()) == c.rows
    kept = p.token_to_row >= 0
    assert np.array_equal(p.token_to_row[kept], (idx * cap + p.slot)[kept])
    assert np.all(p.token_to_row[~kept] == -1)
    for e in range(n):
        lo, hi = c.expert_offsets[e], c.expert_offsets[e + 1]
        assert np.array_equal(p.row_to_token[e * cap:e * cap + hi - lo], c.row_to_token[lo:hi])
        assert np.all(p.row_to_token[e * cap + hi - lo:(e + 1) * cap] == -1)
    # the dispatched buffers agree on every filled row
    x = np.arange(T * 3, dtype=np.float32).reshape(T, 3)
    bc, bp = D.dispatch_rows(x, c), D.dispatch_rows(x, p)
    for e in range(n):
        lo, hi = c.expert_offsets[e], c.expert_offsets[e + 1]
        assert np.array_equal(bp[e * cap:e * cap + hi - lo], bc[lo:hi])


# ---------------------------------------------------------------- expert FFN + combine
def test_bf16_round_matches_torch_rne_on_fp32_values():
    g = np.random.default_rng(0)
    v = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20]
    ours = E.to_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    r = E.bf16_round(v[:4].astype(np.float64))
    assert r.tolist() == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]


def test_relu_ffn_identity_weights_is_relu():
    d = 32
    g = np.random.default_rng(1)
    x = E.bf16_round(g.standard_normal((5, d)))
    eye = E.to_bf16_bits(np.eye(d))
    y = E.relu_ffn(x, eye, eye)
    np.testing.assert_array_equal(y, np.maximum(x, 0.0))
    neg = E.to_bf16_bits(-np.eye(d))
    np.testing.assert_array_equal(E.relu_ffn(x, eye, neg), -np.maximum(x, 0.0))
    # W1 = 2I, W2 = I/4: x -> relu(2x)/4 = relu(x)/2 exactly (powers of two)
    y2 = E.relu_ffn(x, E.to_bf16_bits(2 * np.eye(d)), E.to_bf16_bits(0.25 * np.eye(d)))
    np.testing.assert_array_equal(y2, np.maximum(x, 0.0) / 2)


def test_relu_ffn_hidden_rounding_happens():
    # hidden = 1 + 2^-9 rounds to 1 in bf16 before the second matmul
    x = np.array([[1.0, 2 ** -9]])
    w1 = E.to_bf16_bits(np.array([[1.0, 1.0]]))          # d_ff = 1, d = 2
    w2 = E.to_bf16_bits(np.array([[1.0]]))               # d = 1 output
    assert E.relu_ffn(x, w1, w2).tolist() == [[1.0]]


def test_combine_identity_expert():
    T, d, n = 40, 8, 4
    g = np.random.default_rng(2)
    x = g.standard_normal((T, d))
    idx = g.integers(0, n, (T, 1)).astype(np.int32)
    dm = D.dispatch_maps(idx, n, cap=6)
    y = x[dm.row_to_token]
    gate = g.random((T, 1))
    out = E.combine(x, y, gate, dm.token_to_row)
    kept = dm.token_to_row[:, 0] >= 0
    np.testing.assert_allclose(out[kept], (1 + gate[kept]) * x[kept], rtol=1e-15)
    assert np.array_equal(out[~kept], x[~kept])          # dropped: residual only, bit-exact
    out1 = E.combine(x, y, np.ones((T, 1)), dm.token_to_row)
    np.testing.assert_array_equal(out1[kept], 2 * x[kept])
    branch = E.combine(x, y, gate, dm.token_to_row, residual=False)
    assert np.all(branch[~kept] == 0)
