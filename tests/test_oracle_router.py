"""Pins of the router oracle against facts the pages and mathematics fix (CPU only)."""
import numpy as np
import pytest
import scipy.special

import workloads as W
from oracle import router as R
from oracle import stats as S


def test_softmax_matches_scipy_and_sums_to_one():
    g = np.random.default_rng(0)
    h = g.standard_normal((64, 37)) * 3
    p = R.softmax(h)
    np.testing.assert_allclose(p, scipy.special.softmax(h, axis=1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)


def test_zero_router_gives_uniform_probs():
    """W_r = 0: every logit is 0, so p_i = 1/N exactly (Step 1 of the Switch routing)."""
    x = W.switch_inputs(W.TINY_SWITCH, 0).x
    w = np.zeros((x.shape[1], 8), np.float32)
    rt = R.route(x, w, 1)
    assert np.all(rt.probs == 1.0 / 8)
    assert np.all(rt.idx[:, 0] == 0)          # all tied: lower index wins
    np.testing.assert_allclose(rt.gate, 1.0 / 8)


def test_argmax_of_logits_equals_argmax_of_probs():
    inp = W.switch_inputs(W.TINY_SWITCH, 1)
    rt = R.route(inp.x, inp.w_r, 1)
    h = R.logits(inp.x, inp.w_r)
    assert np.array_equal(np.argmax(rt.probs, axis=1), rt.idx[:, 0])
    assert np.array_equal(np.argmax(h, axis=1), rt.idx[:, 0])


def _brute_topk(keys, k):
    out = []
    for row in keys:
        taken = []
        for _ in range(k):
            best = None
            for j, v in enumerate(row):
                if j in taken:
                    continue
                if best is None or v > row[best]:      # strict: earlier index wins ties
                    best = j
            taken.append(best)
        out.append(taken)
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_matches_brute_force_with_ties(k):
    g = np.random.default_rng(k)
    keys = np.round(g.random((50, 7)) * 3) / 3       # quantised: many ties
    assert np.array_equal(R.topk(keys, k), _brute_topk(keys, k))


def test_topk_hand_example():
    keys = np.array([[0.1, 0.9, 0.5, 0.9],
                     [2.0, -1.0, 3.0, 0.0],
                     [0.0, 0.0, 0.0, 0.0]])
    assert R.topk(keys, 2).tolist() == [[1, 3], [2, 0], [0, 1]]


def test_switch_gate_is_max_probability():
    inp = W.switch_inputs(W.TINY_SWITCH, 2)
    rt = R.route(inp.x, inp.w_r, 1)
    np.testing.assert_allclose(rt.gate[:, 0], rt.probs.max(axis=1), rtol=1e-15)
    h = R.logits(inp.x, inp.w_r)
    np.testing.assert_allclose(rt.gate[:, 0], 1.0 / np.exp(h - h.max(axis=1, keepdims=True)).sum(axis=1),
                               rtol=1e-13)


def test_lossfree_bias_ranks_but_does_not_gate():
    """eq. (1): the bias only reorders experts; the gate stays sigmoid(h)."""
    x = np.eye(3, dtype=np.float32)                   # token i sees logit row i of W_r
    w = np.array([[2.0, 1.0, 0.0],
                  [0.0, 1.0, 3.0],
                  [1.0, 1.0, 1.0]], np.float32)
    bias = np.array([0.0, 0.2, 0.0], np.float32)
    rt = R.route(x, w, 1, score="sigmoid", bias=bias)
    sig = 1 / (1 + np.exp(-w.astype(np.float64)))
    # token 0: sigmoid(2)=0.881 < sigmoid(1)+0.2=0.931 -> expert 1; token 1: sigmoid(3)=0.953 wins
    assert rt.idx[:, 0].tolist() == [1, 2, 1]
    np.testing.assert_allclose(rt.gate[:, 0], [sig[0, 1], sig[1, 2], sig[2, 1]], rtol=1e-15)
    rt0 = R.route(x, w, 1, score="sigmoid")
    assert rt0.idx[:, 0].tolist() == [0, 2, 0]


def test_renorm_gate_sums_to_one():
    inp = W.switch_inputs(W.TINY_SWITCH.scaled(N=8), 3)
    rt = R.route(inp.x, inp.w_r, 3, gate="renorm")
    np.testing.assert_allclose(rt.gate.sum(axis=1), 1.0, rtol=1e-14)
    # equals Softmax over the top-k logits (Shazeer top-k gating)
    h = R.logits(inp.x, inp.w_r)
    hk = np.take_along_axis(h, rt.idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(rt.gate, scipy.special.softmax(hk, axis=1), rtol=1e-13)


def test_near_tie_margin():
    keys = np.array([[1.0, 1.0 - 5e-7, 0.0],       # gap 5e-7 relative to 1 -> near tie
                     [1.0, 0.5, 0.0],
                     [0.3, 0.2, 0.1]])
    m = R.near_tie_margin(keys, 1)
    assert m[0] < 1e-6 and m[1] == pytest.approx(0.5) and m[2] == pytest.approx(1 / 3)
    m2 = R.near_tie_margin(keys, 2)
    assert m2[2] == pytest.approx(1 / 3)
    assert np.all(np.isinf(R.near_tie_margin(keys, 3)) | (R.near_tie_margin(keys, 3) >= 0))


def test_route_counts_sum_to_tokens_times_k():
    inp = W.switch_inputs(W.TINY_SWITCH, 4)
    for k in (1, 2, 4):
        rt = R.route(inp.x, inp.w_r, k)
        assert rt.counts.sum() == inp.x.shape[0] * k
        assert np.all(np.sort(rt.idx, axis=1)[:, 1:] != np.sort(rt.idx, axis=1)[:, :-1])  # distinct


def test_bf16_hidden_decoded_exactly():
    bits = np.array([0x3F80, 0xBF80, 0x3F81, 0x0000, 0x4049], np.uint16)
    v = R.decode_hidden(bits)
    assert v.tolist() == [1.0, -1.0, 1.0 + 2 ** -7, 0.0, 3.140625]
