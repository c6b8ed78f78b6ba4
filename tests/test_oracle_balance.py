"""Pins of the balanced-assignment oracle (QB duals, exact completion) — CPU only."""
import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment

import workloads as W
from oracle import balance as B
from oracle import stats as S


def tiny_scores(seed, m=12, n=4):
    return W.balanced_scores(W.BalancedSpec(m=m, n=n, k=2), seed)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny_lp(seed):
    """m=12, n=4, k=2: both exhaustive methods count the feasible assignments
    (12x4 binary matrices with row sums 2 and column sums 6) and find the
    optimum; the LP (eq. 4), the exact completion and QB+completion agree."""
    s = tiny_scores(seed)
    cnt_dp, best_dp = B.brute_force_dp(s, 2)
    cnt_mm, best_mm, x_mm = B.brute_force_mitm(s, 2)
    assert cnt_dp == cnt_mm == 32496156
    assert best_dp == pytest.approx(best_mm, abs=1e-9)
    xl, obj = B.lp_highs(s, 2)
    assert obj == pytest.approx(best_dp, abs=1e-7)
    comp = B.ssp_complete(s, 2, np.zeros(4, np.float32))
    assert np.array_equal(comp.x, x_mm)
    assert B.objective(s, comp.x) == pytest.approx(best_dp, abs=1e-9)
    _, beta, _ = B.qb_solve(s, 2, 3)
    comp2 = B.ssp_complete(s, 2, beta)
    assert np.array_equal(comp2.x, x_mm)


def test_lp_relaxation_is_integral_and_matches_completion():
    """"극대-극소": the relaxation's optimum is a 0/1 assignment."""
    spec = W.BalancedSpec(m=256, n=16, k=2)
    s = W.balanced_scores(spec, 3)
    xl, obj = B.lp_highs(s, 2)
    frac = np.minimum(np.abs(xl), np.abs(1 - xl))
    assert frac.max() < 1e-7
    comp = B.ssp_complete(s, 2, np.zeros(16, np.float32))
    assert np.array_equal(comp.x, xl > 0.5)
    assert comp.x.sum(axis=0).tolist() == [spec.q] * 16
    assert comp.x.sum(axis=1).tolist() == [2] * 256


@pytest.mark.parametrize("seed", [0, 1])
def test_k1_reduces_to_linear_sum_assignment(seed):
    """k = 1, n | m: replicate each expert q times -> an m x m assignment problem."""
    m, n = 64, 8
    s = W.balanced_scores(W.BalancedSpec(m=m, n=n, k=1), seed)
    q = m // n
    big = np.repeat(s.astype(np.float64), q, axis=1)
    r, c = linear_sum_assignment(big, maximize=True)
    lsa_obj = big[r, c].sum()
    x_lsa = np.zeros((m, n), bool)
    x_lsa[r, c // q] = True
    comp = B.ssp_complete(s, 1, np.zeros(n, np.float32))
    assert B.objective(s, comp.x) == pytest.approx(lsa_obj, abs=1e-9)
    assert np.array_equal(comp.x, x_lsa)


@pytest.mark.parametrize("iters", [0, 1, 5])
def test_dual_certificate(iters):
    """eq. (8) at the completion's potentials equals the primal optimum (strong duality)."""
    spec = W.BalancedSpec(m=512, n=16, k=4)
    s = W.balanced_scores(spec, 4)
    _, beta, _ = B.qb_solve(s, spec.k, iters)
    comp = B.ssp_complete(s, spec.k, beta)
    primal = B.objective(s, comp.x)
    a = B.best_alpha(s, comp.beta, spec.k)
    dual = B.dual_objective(s, a, comp.beta, spec.k)
    assert dual == pytest.approx(primal, rel=1e-12)
    # weak duality at arbitrary duals
    assert B.dual_objective(s, B.best_alpha(s, beta, spec.k), beta, spec.k) >= primal - 1e-9
    # complementary slackness: chosen entries have s - beta >= alpha
    r = s.astype(np.float64) - comp.beta[None, :] - a[:, None]
    assert np.all(r[comp.x] >= -1e-9) and np.all(r[~comp.x] <= 1e-9)


def test_alpha_closed_form_by_scanning_eq10():
    """eq. (10): k·α + Σ_j max(0, v_j − α) is minimal exactly on [v_(k+1), v_(k)]."""
    g = np.random.default_rng(5)
    for k in (1, 2, 3):
        v = g.standard_normal(6)
        srt = -np.sort(-v)
        grid = np.linspace(srt[-1] - 1, srt[0] + 1, 20001)
        f = k * grid + np.maximum(0, v[None, :] - grid[:, None]).sum(axis=1)
        fmin = f.min()
        flat = grid[f <= fmin + 1e-12]
        assert flat.min() >= srt[k] - 1e-3 and flat.max() <= srt[k - 1] + 1e-3
        fa = k * srt[k] + np.maximum(0, v - srt[k]).sum()     # QB's convention: (k+1)-th
        assert fa == pytest.approx(fmin, abs=1e-9)
        a = B.qb_alpha(v[None, :].astype(np.float32), np.zeros(6, np.float32), k)
        assert a[0] == np.float32(srt[k])


def test_qb_order_statistics_are_exact():
    spec = W.BalancedSpec(m=256, n=16, k=3)
    s = W.balanced_scores(spec, 6)
    idx, beta, _ = B.qb_solve(s, spec.k, 2)
    alpha = B.qb_alpha(s, beta, spec.k)
    v = (s - beta[None, :]).astype(np.float32)
    assert np.all((v > alpha[:, None]).sum(axis=1) <= spec.k)
    assert np.all((v >= alpha[:, None]).sum(axis=1) >= spec.k + 1)
    assert np.all(np.any(v == alpha[:, None], axis=1))
    beta2 = B.qb_beta(s, alpha, spec.q)
    w = (s - alpha[:, None]).astype(np.float32)
    assert np.all((w > beta2[None, :]).sum(axis=0) <= spec.q)
    assert np.all((w >= beta2[None, :]).sum(axis=0) >= spec.q + 1)
    assert np.all(np.any(w == beta2[None, :], axis=0))
    assert np.array_equal(idx, np.argsort(-v, axis=1, kind="stable")[:, :spec.k])


def test_qb_online_routes_with_old_beta():
    spec = W.BalancedSpec(m=128, n=8, k=2)
    s = W.balanced_scores(spec, 7)
    beta_old = np.linspace(-1, 1, 8).astype(np.float32)
    idx, beta_new, _ = B.qb_online(s, 2, beta_old)
    assert np.array_equal(idx, B.topk_biased(s, beta_old, 2))
    assert not np.array_equal(idx, B.topk_biased(s, beta_new, 2))
    _, b1, _ = B.qb_solve(s, 2, 1, beta0=beta_old)
    assert np.array_equal(beta_new, b1)


def test_qb_fixed_point_is_lp_optimal():
    """"교대 반복": once QB's x meets both constraint sets it is the LP optimum."""
    hits = 0
    for seed in range(40):
        spec = W.BalancedSpec(m=32, n=4, k=1, offset_std=0.1)
        s = W.balanced_scores(spec, seed)
        idx, beta, _ = B.qb_solve(s, 1, 30)
        x = B.idx_to_x(idx, 4)
        if np.all(x.sum(axis=0) == spec.q):
            hits += 1
            comp = B.ssp_complete(s, 1, np.zeros(4, np.float32))
            assert np.array_equal(x, comp.x)
    assert hits >= 2


def test_qb_improves_balance_on_demo_workload():
    """"데모 코드": subtracting the QB bias lowers the max violation."""
    s = W.uniform_offset_scores(4000, 64, 0)
    k = 4
    top = np.argsort(-s, axis=1)[:, :k]
    before = S.load_violation(np.bincount(top.ravel(), minlength=64))
    idx, beta, _ = B.qb_solve(s, k, 5)
    after = S.load_violation(np.bincount(idx.ravel(), minlength=64))
    assert after[0] < 0.25 * before[0] and after[2] < 0.25 * before[2]


def test_qb_quantile_is_the_type7_sample_quantile():
    """The demo's quantile on each axis is the order statistic at position (N − 1)(1 − k/n)
    linearly interpolated with the next one: checked against np.interp over the sorted values
    (float64), to fp32 rounding, and against the exact-mode neighbours it lies between."""
    s = W.uniform_offset_scores(3008, 64, 3)   # m k / n = 188 whole, so the column bracket is (q+1)-th, q-th
    k, n = 4, 64
    beta = np.linspace(-0.2, 0.3, n).astype(np.float32)
    a = B.quantile_alpha(s, beta, k)
    v = (s - beta[None, :]).astype(np.float32).astype(np.float64)
    p = (n - 1) * (1 - k / n)
    ref = np.array([np.interp(p, np.arange(n), np.sort(r)) for r in v])
    np.testing.assert_allclose(a, ref, rtol=2e-7, atol=1e-7)
    lo, hi = B.qb_alpha(s, beta, k), B.qb_alpha(s, beta, k - 1)     # (k+1)-th and k-th largest
    assert np.all((a >= lo) & (a <= hi))
    b = B.quantile_beta(s, a, k)
    w = (s - a[:, None]).astype(np.float32).astype(np.float64)
    m, q = s.shape[0], s.shape[0] * k // n
    pc = (m - 1) * (1 - k / n)
    refc = np.array([np.interp(pc, np.arange(m), np.sort(w[:, j])) for j in range(n)])
    np.testing.assert_allclose(b, refc, rtol=2e-7, atol=1e-7)
    assert np.all((b >= B.qb_beta(s, a, q)) & (b <= B.qb_beta(s, a, q - 1)))


def test_qb_quantile_balances_the_demo_workload_and_bip_clips():
    """The demo itself at m = 100000, n = 256, k = 8, T = 5: the max and mean violation of the
    biased top-k fall far below those of the plain top-k; the BIP clip keeps α, β >= 0 and
    changes nothing where they are positive anyway."""
    m, n, k = 100000, 256, 8
    s = W.uniform_offset_scores(m, n, 0)
    top = np.argsort(-s, axis=1)[:, :k]
    before = S.load_violation(np.bincount(top.ravel(), minlength=n))
    idx, beta, alpha = B.qb_quantile_solve(s, k, 5)
    after = S.load_violation(np.bincount(idx.ravel(), minlength=n))
    assert before[0] > 0.5 and after[0] < 0.05 * before[0] and after[2] < 0.05 * before[2]
    _, bb, ab = B.qb_quantile_solve(s, k, 5, bip=True)
    assert np.all(bb >= 0) and np.all(ab >= 0)
    if np.all(alpha > 0) and np.all(beta > 0):
        assert np.array_equal(bb, beta)


@pytest.mark.slow
def test_full_size_completion_matches_highs():
    """The balanced-LP workload at full size (m=4096, n=64, k=4)."""
    spec = W.BALANCED
    s = W.balanced_scores(spec, 0)
    _, beta, _ = B.qb_solve(s, spec.k, 20)
    comp = B.ssp_complete(s, spec.k, beta)
    xl, obj = B.lp_highs(s, spec.k)
    assert np.array_equal(comp.x, xl > 0.5)
    assert B.objective(s, comp.x) == pytest.approx(obj, rel=1e-12)


# ------------------------------------------------------------------ SignSGD on β (eq. (15)-(17))
def test_signsgd_gradient_is_dual_slope():
    # ∂ℓ/∂β_j = q − c_j: central differences of the dual ℓ(β) at a generic β, small
    # enough that no row's top-k changes, equal q − c_j exactly (ℓ is piecewise linear)
    rng = np.random.default_rng(3)
    m, n, k = 240, 12, 3
    s = rng.standard_normal((m, n)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(n)).astype(np.float32)
    c = np.bincount(B.topk_biased(s, beta, k).ravel(), minlength=n)
    q = m * k // n
    for j in range(n):
        e = np.zeros(n)
        e[j] = 1e-7
        d = (B.dual_of_beta(s, beta + e, k) - B.dual_of_beta(s, beta - e, k)) / 2e-7
        assert abs(d - (q - c[j])) < 1e-3


def test_signsgd_step_and_progress():
    rng = np.random.default_rng(4)
    m, n, k, gamma = 4096, 32, 2, 0.01
    s = (rng.random((m, n)) + rng.random(n)[None, :]).astype(np.float32)
    q = m * k // n
    _, b1, _ = B.signsgd_solve(s, k, 1, gamma)
    c0 = np.bincount(B.topk_biased(s, np.zeros(n, np.float32), k).ravel(), minlength=n)
    # one step from 0: overloaded experts up by γ, underloaded down, balanced ones unchanged
    assert np.array_equal(b1, (np.float32(gamma) * np.sign(c0 - q)).astype(np.float32))
    # many steps: the violation falls well below the plain top-k's
    vio = lambda c: (c / c.sum() * n - 1).max()
    _, _, c200 = B.signsgd_solve(s, k, 200, gamma)
    assert vio(c200) < 0.25 * vio(c0)


# ------------------------------------------------------------------ BIP (eqs. (12)-(14))
def test_bip_hand_example():
    """m=4, n=2, k=1, q=2 worked by hand.  Row differences from β = 0: the second largest of
    each row is the negative expert-1 score, so every α is truncated to 0.  Column 0 then
    holds 1, 2, 3, 4: its 3rd largest is 2.  Column 1 holds −3, −2, −1, −4: its 3rd largest
    is −3, truncated to β_1 = 0 exactly.  A second step changes nothing (the second largest
    of each row of s − β is still negative).  Without the truncation α = s_·1 and
    β = (4, 0).  The inequality LP assigns tokens 2 and 3 to expert 0 and leaves 0 and 1
    empty; the reduced-cost rule of eq. (7) at the BIP duals gives the same."""
    s = np.array([[1, -3], [2, -2], [3, -1], [4, -4]], np.float32)
    for iters in (1, 2):
        idx, beta, alpha = B.qb_solve(s, 1, iters, bip=True)
        assert alpha.tolist() == [0, 0, 0, 0]
        assert beta.tolist() == [2, 0]
    _, beta_eq, alpha_eq = B.qb_solve(s, 1, 1)
    assert alpha_eq.tolist() == [-3, -2, -1, -4] and beta_eq.tolist() == [4, 0]
    x = B.bip_reduced_assignment(s, np.zeros(4), np.array([2.0, 0.0]))
    assert x.astype(int).tolist() == [[0, 0], [0, 0], [1, 0], [1, 0]]
    xl, obj = B.lp_highs_leq(s, 1)
    assert np.array_equal(xl > 0.5, x) and obj == pytest.approx(7.0)
    # the online form takes the same truncated steps after routing with the old β
    idx_o, beta_o, alpha_o = B.qb_online(s, 1, np.zeros(2, np.float32), bip=True)
    assert beta_o.tolist() == [2, 0] and idx_o[:, 0].tolist() == [0, 0, 0, 0]


def test_bip_fixed_point_is_inequality_lp_optimum():
    """Where the truncated iteration stops moving and its eq. (7) assignment satisfies the
    conditions of the inequality LP (row sums ≤ k, column sums ≤ q, rows with α_i > 0 full,
    columns with β_j > 0 full), that assignment is the optimum of eq. (12)'s relaxation, as
    HiGHS finds it.  Scores of mixed sign make the truncation bite (many zero duals and rows
    left empty)."""
    hits = clipped = 0
    for seed in range(60):
        rng = np.random.default_rng(seed)
        m, n, k = 16, 4, 1
        q = m * k // n
        s = (rng.standard_normal((m, n)) + rng.standard_normal(n) - 0.5).astype(np.float32)
        beta = np.zeros(n, np.float32)
        alpha = np.zeros(m, np.float32)
        for _ in range(60):
            a2 = B.qb_alpha(s, beta, k, bip=True)
            b2 = B.qb_beta(s, a2, q, bip=True)
            if np.array_equal(a2, alpha) and np.array_equal(b2, beta):
                break
            alpha, beta = a2, b2
        else:
            continue
        assert np.all(alpha >= 0) and np.all(beta >= 0)
        x = B.bip_reduced_assignment(s, alpha, beta)
        r, c = x.sum(axis=1), x.sum(axis=0)
        if not (np.all(r <= k) and np.all(c <= q) and np.all(r[alpha > 0] == k) and np.all(c[beta > 0] == q)):
            continue
        hits += 1
        clipped += int(np.any(alpha == 0) and r.sum() < m * k)
        xl, _ = B.lp_highs_leq(s, k)
        assert np.array_equal(x, xl > 0.5)
    assert hits >= 10 and clipped >= 10


# ------------------------------------------------------------------ mini-batch β ("함정에 주의")
def test_minibatch_beta_hand_example():
    """Two mini-batches of two tokens, n=2, k=1 (q_b = 1), one step from β = 0.
    Batch A = [[5, 1], [4, 0]]: α = (1, 0), columns of s − α are (4, 4) and (0, 0), so
    β_A = (4, 0).  Batch B = [[1, 3], [2, 7]]: α = (1, 2), columns (0, 0) and (2, 5), so
    β_B = (0, 2).  The mean is (2, 1).  One selection over all four tokens (q = 2) gives
    (0, 0) instead."""
    s = np.array([[5, 1], [4, 0], [1, 3], [2, 7]], np.float32)
    assert B.minibatch_beta(s, 1, 1, 2).tolist() == [2.0, 1.0]
    assert B.qb_solve(s, 1, 1)[1].tolist() == [0.0, 0.0]
    with pytest.raises(ValueError):
        B.minibatch_beta(s, 1, 1, 3)


@pytest.mark.parametrize("iters,bip", [(1, False), (3, False), (2, True)])
def test_minibatch_beta_reductions(iters, bip):
    """One mini-batch is the plain solve; identical mini-batches average to that block's β."""
    spec = W.BalancedSpec(m=256, n=16, k=2)
    s = W.balanced_scores(spec, 8)
    beta0 = np.linspace(-0.3, 0.3, 16).astype(np.float32)
    assert np.array_equal(B.minibatch_beta(s, 2, iters, 256, beta0, bip), B.qb_solve(s, 2, iters, beta0, bip)[1])
    block = s[:64]
    tiled = np.concatenate([block] * 4)
    assert np.array_equal(B.minibatch_beta(tiled, 2, iters, 64, beta0, bip), B.qb_solve(block, 2, iters, beta0, bip)[1])
    # the quantile form likewise
    assert np.array_equal(B.minibatch_beta(s, 2, iters, 256, beta0, bip, quantile=True),
                          B.qb_quantile_solve(s, 2, iters, bip, beta0)[1])
    assert np.array_equal(B.minibatch_beta(tiled, 2, iters, 64, beta0, bip, quantile=True),
                          B.qb_quantile_solve(block, 2, iters, bip, beta0)[1])


def test_quantile_helper_equals_numpy_on_fp32():
    """The interpolation rule written out in _interp_quantile_fp32 reproduces numpy's quantile
    on fp32 data bit for bit (a library routine; levels with weight below and above 1/2, and
    a level at the top)."""
    rng = np.random.default_rng(9)
    for N, level in [(256, 1 - 8 / 256), (100000, 1 - 8 / 256), (64, 1 - 4 / 64), (7, 0.3), (10, 0.95),
                     (5, 1.0), (33, 0.5)]:
        v = rng.standard_normal((N, 3)).astype(np.float32)
        got = B._interp_quantile_fp32(np.sort(v, axis=0), np.float32(level))
        ref = np.quantile(v, level, axis=0)
        assert ref.dtype == np.float32
        assert np.array_equal(got, ref), (N, level)
