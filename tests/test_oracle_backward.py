"""Pins of the backward-pass oracle (CPU only): central differences of the layer's scalar loss,
written directly from the forward definitions, and closed forms."""
import numpy as np
import pytest

from oracle import backward as B
from oracle import dispatch as OD
from oracle import router as R


def _instance(seed, T=24, d=8, N=4, k=1, d_ff=6, cap=5, alpha=0.1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, N)) * 0.5
    w1 = rng.standard_normal((N, d_ff, d)) * 0.4
    w2 = rng.standard_normal((N, d, d_ff)) * 0.4
    dout = rng.standard_normal((T, d))
    idx = R.topk(x @ w_r, k)
    dm = OD.dispatch_maps(idx, N, cap, padded=True)
    counts = np.bincount(idx.ravel(), minlength=N)
    return x, w_r, w1, w2, dout, idx, dm, counts, alpha


@pytest.mark.parametrize("seed,k,cap", [(0, 1, 5), (1, 1, 3), (2, 2, 9), (3, 2, 4)])
def test_gradients_match_central_differences(seed, k, cap):
    x, w_r, w1, w2, dout, idx, dm, counts, alpha = _instance(seed, k=k, cap=cap)
    assert dm.drop_mask.sum() > 0 or cap >= 9          # some cases drop pairs
    g = B.switch_layer_backward(x, w_r, idx, dm.token_to_row, dm.expert_offsets, dm.expert_rows, w1, w2, dout,
                                alpha, counts=counts, rounded=False)
    loss = lambda x_, wr_, w1_, w2_: B.switch_layer_loss(x_, wr_, idx, dm.token_to_row, dm.expert_offsets,  # noqa
                                                        dm.expert_rows, w1_, w2_, dout, alpha, counts)
    eps = 1e-6
    rng = np.random.default_rng(100 + seed)
    for name, arr, grad in (("x", x, g.dx), ("w_r", w_r, g.dw_r), ("w1", w1, g.dw1), ("w2", w2, g.dw2)):
        for _ in range(12):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += eps
            am[pos] -= eps
            args_p = {"x": (ap, w_r, w1, w2), "w_r": (x, ap, w1, w2), "w1": (x, w_r, ap, w2),
                      "w2": (x, w_r, w1, ap)}[name]
            args_m = {"x": (am, w_r, w1, w2), "w_r": (x, am, w1, w2), "w1": (x, w_r, am, w2),
                      "w2": (x, w_r, w1, am)}[name]
            num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert grad[pos] == pytest.approx(num, rel=1e-5, abs=1e-7), (name, pos)


def test_balancing_loss_gradient_closed_form():
    """W_r = 0 gives p = 1/N for every token; with no upstream gradient only the balancing loss
    acts: dh_j(t) = (c_j − mean(c)) / N with c_j = α·N·f_j/T, so dW_r = xᵀ·dh = (Σ_t x_t)(c − c̄)ᵀ / N."""
    T, d, N, alpha = 16, 5, 4, 0.01
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, d))
    idx = np.array([[0]] * 7 + [[1]] * 5 + [[3]] * 4)
    counts = np.bincount(idx.ravel(), minlength=N)
    dm = OD.dispatch_maps(idx, N, 8, padded=True)
    w1 = np.zeros((N, 3, d))
    w2 = np.zeros((N, d, 3))
    g = B.switch_layer_backward(x, np.zeros((d, N)), idx, dm.token_to_row, dm.expert_offsets, dm.expert_rows,
                                w1, w2, np.zeros((T, d)), alpha, counts=counts, rounded=False)
    c = alpha * N * (counts / T) / T
    np.testing.assert_allclose(g.dh, np.tile((c - c.mean()) / N, (T, 1)), rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(g.dw_r, np.outer(x.sum(axis=0), (c - c.mean()) / N), rtol=1e-12, atol=1e-18)
    assert np.all(g.dx == 0)        # dx_router = dh·W_rᵀ = 0 with W_r = 0, and dout = 0


def test_dropped_tokens_get_only_residual_and_router_gradients():
    x, w_r, w1, w2, dout, idx, dm, counts, alpha = _instance(4, cap=2)
    g = B.switch_layer_backward(x, w_r, idx, dm.token_to_row, dm.expert_offsets, dm.expert_rows, w1, w2, dout,
                                alpha, counts=counts, rounded=False)
    dropped = dm.drop_mask[:, 0] == 1
    assert dropped.sum() > 0
    assert np.all(g.dgate[dropped] == 0)
    p = R.softmax(x @ w_r)
    c = alpha * w_r.shape[1] * (counts / x.shape[0]) / x.shape[0]
    dh_drop = p * (c - (p * c).sum(axis=1, keepdims=True))
    np.testing.assert_allclose(g.dh[dropped], dh_drop[dropped], rtol=1e-12)
    np.testing.assert_allclose(g.dx[dropped], dout[dropped] + dh_drop[dropped] @ w_r.T, rtol=1e-12)
