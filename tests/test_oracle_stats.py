"""Pins of the statistics / aux-loss / Loss-Free oracle (CPU only)."""
import numpy as np
import pytest

import workloads as W
from oracle import router as R
from oracle import stats as S


def cyclic_balanced_inputs(T, N, d):
    """Token t sees logits = v shifted cyclically by t, with W_r = [I_N; 0].

    Over T = multiple of N tokens every expert is chosen T/N times and every
    expert's mean probability is 1/N (each probability vector is a permutation
    of the same vector, and the permutations cover every rotation equally).
    """
    assert T % N == 0 and d >= N
    v = np.linspace(1.0, -1.0, N).astype(np.float32)
    x = np.zeros((T, d), np.float32)
    for t in range(T):
        x[t, :N] = np.roll(v, t)
    w = np.zeros((d, N), np.float32)
    w[:N, :N] = np.eye(N, dtype=np.float32)
    return x, w


@pytest.mark.parametrize("T,N,d", [(64, 8, 16), (256, 16, 16), (1024, 8, 64)])
def test_balanced_case_gives_aux_equal_alpha(T, N, d):
    """"로드 밸런싱 손실": f_i = P_i = 1/N gives L_aux = α."""
    x, w = cyclic_balanced_inputs(T, N, d)
    rt = R.route(x, w, 1)
    f, P, aux = S.switch_stats(rt.counts, rt.prob_sum, T, 1e-2)
    np.testing.assert_array_equal(f, np.full(N, 1.0 / N))
    np.testing.assert_allclose(P, 1.0 / N, rtol=1e-12)
    assert aux == pytest.approx(1e-2, rel=1e-12)


def test_uniform_router_gives_alpha_for_any_counts():
    x = W.switch_inputs(W.TINY_SWITCH, 0).x
    rt = R.route(x, np.zeros((64, 8), np.float32), 1)
    f, P, aux = S.switch_stats(rt.counts, rt.prob_sum, 1024, 1e-2)
    assert f[0] == 1.0 and aux == pytest.approx(1e-2, rel=1e-14)


def test_aux_hand_example():
    f, P, aux = S.switch_stats(np.array([3, 1]), np.array([2.4, 1.6]), 4, 0.01)
    assert f.tolist() == [0.75, 0.25]
    assert P.tolist() == [0.6, 0.4]
    assert aux == pytest.approx(0.01 * 2 * (0.75 * 0.6 + 0.25 * 0.4), rel=1e-15)
    assert aux == pytest.approx(0.011, rel=1e-14)


def test_aux_skewed_is_larger_than_balanced():
    # all tokens to expert 0 with P concentrated there: aux = α·N
    f, P, aux = S.switch_stats(np.array([10, 0, 0, 0]), np.array([10.0, 0, 0, 0]), 10, 0.01)
    assert aux == pytest.approx(0.04)


def test_global_batch_reduces_to_switch_for_one_micro_batch():
    inp = W.switch_inputs(W.TINY_SWITCH, 5)
    rt = R.route(inp.x, inp.w_r, 1)
    gb = S.GlobalBatch(8)
    gb.add(rt.counts, 1024, rt.prob_sum)
    f, P, aux = S.switch_stats(rt.counts, rt.prob_sum, 1024, 1e-2)
    assert gb.loss(1e-2) == pytest.approx(aux, rel=1e-14)
    # identical micro-batches: global loss equals the per-micro-batch loss
    gb2 = S.GlobalBatch(8)
    for _ in range(4):
        gb2.add(rt.counts, 1024, rt.prob_sum)
    assert gb2.loss(1e-2) == pytest.approx(aux, rel=1e-14)
    np.testing.assert_array_equal(gb2.counts, 4 * rt.counts)


def test_global_batch_differs_from_micro_when_domains_skew():
    """Two micro-batches that each load one expert: micro-batch losses see the skew,
    the global f is balanced (the point of [Qwen global])."""
    gb = S.GlobalBatch(2)
    gb.add(np.array([4, 0]), 4, np.array([3.0, 1.0]))
    gb.add(np.array([0, 4]), 4, np.array([1.0, 3.0]))
    np.testing.assert_array_equal(gb.f(), [0.5, 0.5])
    micro = [S.switch_stats(np.array([4, 0]), np.array([3.0, 1.0]), 4, 1e-2)[2],
             S.switch_stats(np.array([0, 4]), np.array([1.0, 3.0]), 4, 1e-2)[2]]
    assert gb.loss(1e-2) == pytest.approx(1e-2)          # 0.01·2·(0.5·0.75 + 0.5·0.25)
    assert np.mean(micro) == pytest.approx(0.015)


def test_hybrid_loss_closed_forms():
    """Hybrid = w_g·global + w_m·micro, both readings of the 0.01 weight.  On the skewed pair
    above each micro loss is 0.015 (each micro-batch loads one expert, whose P is 0.75) and
    each global loss 0.01.  Reading A (micro loss weighted 0.01): 0.01 + 0.01·0.015 = 0.01015.
    Reading B (global loss weighted 0.01): 0.01·0.01 + 0.015 = 0.0151.  One micro-batch alone
    has L_global = L_micro = the Switch loss, so hybrid = (w_g + w_m)·aux."""
    gb = S.GlobalBatch(2)
    gb.add(np.array([4, 0]), 4, np.array([3.0, 1.0]))
    gb.add(np.array([0, 4]), 4, np.array([1.0, 3.0]))
    np.testing.assert_allclose(gb.micro_losses(1e-2), [0.015, 0.015], rtol=1e-14)   # 0.01·2·(1·0.75)
    np.testing.assert_allclose(gb.hybrid_losses(1e-2, 1.0, 0.01), [0.01015, 0.01015], rtol=1e-13)
    np.testing.assert_allclose(gb.hybrid_losses(1e-2, 0.01, 1.0), [0.0151, 0.0151], rtol=1e-13)
    assert gb.hybrid_loss(1e-2, 1.0, 0.01) == pytest.approx(0.01015, rel=1e-13)
    assert gb.hybrid_loss(1e-2, 0.01, 1.0) == pytest.approx(0.0151, rel=1e-13)
    inp = W.switch_inputs(W.TINY_SWITCH, 6)
    rt = R.route(inp.x, inp.w_r, 1)
    one = S.GlobalBatch(8)
    one.add(rt.counts, 1024, rt.prob_sum)
    aux = S.switch_stats(rt.counts, rt.prob_sum, 1024, 1e-2)[2]
    assert one.hybrid_loss(1e-2, 1.0, 0.01) == pytest.approx(1.01 * aux, rel=1e-13)
    assert one.hybrid_loss(1e-2, 0.01, 1.0) == pytest.approx(1.01 * aux, rel=1e-13)
    assert one.hybrid_loss(1e-2, 1.0, 0.0) == pytest.approx(aux, rel=1e-14)
    assert one.hybrid_loss(1e-2, 0.0, 1.0) == pytest.approx(aux, rel=1e-14)


def test_lossfree_update_signs_and_fp32_rounding():
    b = np.array([1.0, 0.0, -0.25, 3.0], np.float32)
    c = np.array([9, 8, 7, 8])                            # m*k/n = 8 per expert
    nb = S.lossfree_update(b, c, m=16, k=2, gamma=1e-3)
    g = np.float32(1e-3)
    assert nb.dtype == np.float32
    assert nb[0] == np.float32(np.float32(1.0) - g)     # over-loaded: decreases
    assert nb[1] == np.float32(0.0)                       # balanced: unchanged
    assert nb[2] == np.float32(np.float32(-0.25) + g)    # under-loaded: increases
    assert nb[3] == np.float32(3.0)
    # exactly one fp32 rounding: 1 - fl32(1e-3) is not 0.999 in float64
    assert float(nb[0]) != 0.999 and abs(float(nb[0]) - 0.999) < 1e-7
    # balanced counts keep b bit-identical
    assert np.array_equal(S.lossfree_update(b, np.full(4, 8), 16, 2, 1e-3), b)


def test_lossfree_sign_is_exact_for_huge_batches():
    # F - 1/n in float64 is exactly 0 here (2^55 + 1 rounds to 2^55); the integer test is not
    m, k, n = 2 ** 55, 3, 3
    q = m * k // n
    assert float(q + 1) / float(m * k) - 1 / n == 0.0
    nb = S.lossfree_update(np.zeros(3, np.float32), np.array([q + 1, q, q - 1]), m, k, 1e-3)
    assert nb.tolist() == [-np.float32(1e-3), 0.0, np.float32(1e-3)]


def test_load_violation():
    # balanced: every share is exactly 1/n
    assert S.load_violation(np.full(8, 5)) == (0.0, 0.0, 0.0)
    # hand example: counts 6, 2, 0, 0 -> shares 3/4, 1/4, 0, 0 -> excess 2, 0, -1, -1
    assert S.load_violation(np.array([6, 2, 0, 0])) == (2.0, -1.0, 1.0)
    n, k = 8, 2
    c = np.zeros(n)
    c[:k] = 100
    mx, mn, av = S.load_violation(c)
    assert mx == pytest.approx(n / k - 1) and mn == -1.0
    assert av == pytest.approx((k * (n / k - 1) + (n - k)) / n)
