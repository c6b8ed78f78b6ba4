"""GPU parity: moe_balance_duals (QB solve / online / exact completion), moe_stats,
moe_global_aux and the whole moe_switch_layer against the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import balance as OB
from oracle import dispatch as OD
from oracle import expert as OE
from oracle import router as OR
from oracle import stats as OS
from tests.gpu_util import DEV, assert_rel, check_selection, row_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("load_balanced_expert_amd")


# ------------------------------------------------------------------ balanced assignment
@pytest.mark.parametrize("iters", [1, 5, 20])
def test_qb_solve_bit_exact(iters):
    spec = W.BALANCED
    s = W.balanced_scores(spec, 0)
    say(f"[qb] solve m={spec.m} n={spec.n} k={spec.k} iters={iters}")
    beta = torch.zeros(spec.n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), spec.k, beta, iters=iters)
    torch.cuda.synchronize()
    idx_r, beta_r, alpha_r = OB.qb_solve(s, spec.k, iters)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.alpha), alpha_r)
    assert np.array_equal(to_host(out.idx), idx_r)
    counts = np.bincount(idx_r.ravel(), minlength=spec.n)
    assert np.array_equal(to_host(out.counts), counts)
    info = to_host(out.info)
    assert info[0] == iters and info[2] == int(np.all(counts == spec.q))


@pytest.mark.parametrize("m,n,k", [(1000, 8, 2), (96, 32, 3), (4096, 256, 8)])
def test_qb_solve_other_shapes(m, n, k):
    spec = W.BalancedSpec(m=m, n=n, k=k)
    s = W.balanced_scores(spec, 1)
    beta0 = np.linspace(-0.5, 0.5, n).astype(np.float32)
    beta = to_dev(beta0)
    out = M.balance_duals(to_dev(s), k, beta, iters=3)
    torch.cuda.synchronize()
    idx_r, beta_r, _ = OB.qb_solve(s, k, 3, beta0=beta0)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.idx), idx_r)


@pytest.mark.parametrize("m,n,k,iters,bip", [(4096, 64, 4, 5, False), (3200, 256, 8, 5, False),
                                             (3200, 256, 8, 5, True), (1000, 8, 2, 3, False), (96, 32, 3, 2, True)])
def test_qb_quantile_bit_exact(m, n, k, iters, bip):
    # the demo code's interpolated quantiles on both axes, against numpy's quantile in the oracle
    s = W.uniform_offset_scores(m, n, 11)
    say(f"[qb] quantile m={m} n={n} k={k} iters={iters} bip={bip}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), k, beta, iters=iters, quantile=True, bip=bip)
    torch.cuda.synchronize()
    idx_r, beta_r, alpha_r = OB.qb_quantile_solve(s, k, iters, bip=bip)
    assert np.array_equal(to_host(out.alpha), alpha_r)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.idx), idx_r)


@pytest.mark.parametrize("m,n,k,iters,scores", [(4096, 64, 4, 5, "balanced"), (3200, 256, 8, 3, "mixed"),
                                                (1000, 80, 40, 2, "mixed"), (2000, 320, 4, 3, "mixed")])
def test_qb_bip_exact_form_bit_exact(m, n, k, iters, scores):
    # BIP's truncated steps on exact order statistics ([MoE tour 6] eq. (14)): scores of mixed
    # sign, so that many α and β are truncated to 0
    if scores == "balanced":
        s = W.balanced_scores(W.BalancedSpec(m=m, n=n, k=k), 3)
    else:
        s = (W.uniform_offset_scores(m, n, 13) - np.float32(1.2)).astype(np.float32)
    say(f"[qb] bip exact form m={m} n={n} k={k} iters={iters}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), k, beta, iters=iters, bip=True)
    torch.cuda.synchronize()
    idx_r, beta_r, alpha_r = OB.qb_solve(s, k, iters, bip=True)
    assert np.all(beta_r >= 0) and np.all(alpha_r >= 0)
    if scores == "mixed":
        assert np.any(alpha_r == 0) or np.any(beta_r == 0)   # the truncation is exercised
    assert np.array_equal(to_host(out.alpha), alpha_r)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.idx), idx_r)
    # the online form with the truncation
    beta_old = (np.abs(np.random.default_rng(4).standard_normal(n)) * 0.1).astype(np.float32)
    beta = to_dev(beta_old)
    out = M.balance_duals(to_dev(s), k, beta, iters=1, mode="online", bip=True)
    torch.cuda.synchronize()
    idx_r, beta_r, alpha_r = OB.qb_online(s, k, beta_old, bip=True)
    assert np.array_equal(to_host(out.idx), idx_r)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.alpha), alpha_r)


@pytest.mark.parametrize("m,n,k,batch,iters,quantile,bip", [
    (4096, 64, 4, 1024, 5, False, False),     # the balanced-LP workload in 4 mini-batches
    (4096, 64, 4, 64, 3, False, True),        # 64 mini-batches, truncated steps
    (6400, 256, 8, 1600, 3, True, False),     # the demo's shape, quantile form
    (3200, 320, 4, 640, 2, False, False),     # more than 256 experts (generic row kernel)
    (4096, 64, 4, 4096, 4, False, False),     # one mini-batch: the plain solve
])
def test_minibatch_beta_bit_exact(m, n, k, batch, iters, quantile, bip):
    s = W.uniform_offset_scores(m, n, 17)
    beta0 = np.linspace(-0.1, 0.1, n).astype(np.float32)
    say(f"[qb] mini-batch m={m} n={n} k={k} batch={batch} iters={iters} quantile={quantile} bip={bip}")
    beta = to_dev(beta0)
    out = M.balance_duals_minibatch(to_dev(s), k, beta, batch, iters=iters, quantile=quantile, bip=bip)
    torch.cuda.synchronize()
    beta_r = OB.minibatch_beta(s, k, iters, batch, beta0, bip=bip, quantile=quantile)
    assert np.array_equal(to_host(beta), beta_r)
    idx_r = OB.topk_biased(s, beta_r, k)
    assert np.array_equal(to_host(out.idx), idx_r)
    assert np.array_equal(to_host(out.counts), np.bincount(idx_r.ravel(), minlength=n))
    if batch == m:
        _, beta_p, _ = (OB.qb_quantile_solve(s, k, iters, bip, beta0) if quantile else
                        OB.qb_solve(s, k, iters, beta0, bip))
        assert np.array_equal(beta_r, beta_p)
    # online: route with the old β, then one step per mini-batch from it
    beta = to_dev(beta0)
    out = M.balance_duals_minibatch(to_dev(s), k, beta, batch, iters=1, mode="online", quantile=quantile, bip=bip)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out.idx), OB.topk_biased(s, beta0, k))
    assert np.array_equal(to_host(beta), OB.minibatch_beta(s, k, 1, batch, beta0, bip=bip, quantile=quantile))


@pytest.mark.parametrize("m,n,k,levels", [
    (2000, 100, 5, 0),       # 65..128 experts: two experts per lane in the row kernel
    (1600, 320, 4, 0),       # more than 256 experts: the row kernel's arg-best rounds
    (4096, 64, 4, 4),        # scores on a grid of 4 values: equal heads, lowest expert first
    (120000, 8, 2, 2),       # two score values: the column bin overflows LDS, selected in global passes
    (30002, 6, 3, 0),        # columns longer than LDS holds, length not a multiple of 4: sampled window, scalar loads
    (1000, 80, 40, 0),       # more than 32 picks: the counting top-k on whole-wave rows
])
@pytest.mark.parametrize("quantile", [False, True])
def test_qb_kernel_paths(m, n, k, levels, quantile):
    s = W.uniform_offset_scores(m, n, 5)
    if levels:
        s = (np.floor(s * (levels / 2.0)) / levels).astype(np.float32)
    say(f"[qb] paths m={m} n={n} k={k} levels={levels} quantile={quantile}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), k, beta, iters=3, quantile=quantile)
    torch.cuda.synchronize()
    if quantile:
        idx_r, beta_r, alpha_r = OB.qb_quantile_solve(s, k, 3)
    else:
        idx_r, beta_r, alpha_r = OB.qb_solve(s, k, 3)
    assert np.array_equal(to_host(out.alpha), alpha_r)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.idx), idx_r)
    assert np.array_equal(to_host(out.counts), np.bincount(idx_r.ravel(), minlength=n))


@pytest.mark.parametrize("m,n,k,gamma,iters", [(4096, 32, 2, 0.01, 20), (3200, 256, 8, 1e-3, 10),
                                               (1000, 80, 40, 0.01, 5), (2000, 100, 5, 0.02, 0)])
def test_signsgd_bit_exact(m, n, k, gamma, iters):
    # sign-gradient steps on β against the oracle: β bit-exact, the final top-k and counts exact
    s = W.uniform_offset_scores(m, n, 21)
    say(f"[qb] signsgd m={m} n={n} k={k} gamma={gamma} iters={iters}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    idx, counts = M.balance_signsgd(to_dev(s), k, beta, gamma, iters)
    torch.cuda.synchronize()
    idx_r, beta_r, counts_r = OB.signsgd_solve(s, k, iters, gamma)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(idx), idx_r)
    assert np.array_equal(to_host(counts), counts_r)


def test_qb_quantile_demo_full_size():
    # the page's demo: m = 100000, n = 256, k = 8, s = U(0,1) + U(0,1)_n, T = 5
    m, n, k = 100000, 256, 8
    s = W.uniform_offset_scores(m, n, 0)
    say(f"[qb] quantile demo m={m} n={n} k={k}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), k, beta, iters=5, quantile=True)
    torch.cuda.synchronize()
    idx_r, beta_r, _ = OB.qb_quantile_solve(s, k, 5)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.counts), np.bincount(idx_r.ravel(), minlength=n))


def test_qb_online_routes_before_update():
    spec = W.BALANCED
    s = W.balanced_scores(spec, 2)
    beta_old = (np.random.default_rng(0).standard_normal(spec.n) * 0.5).astype(np.float32)
    beta = to_dev(beta_old)
    out = M.balance_duals(to_dev(s), spec.k, beta, iters=1, mode="online")
    torch.cuda.synchronize()
    idx_r, beta_r, alpha_r = OB.qb_online(s, spec.k, beta_old)
    assert np.array_equal(to_host(out.idx), idx_r)
    assert np.array_equal(to_host(beta), beta_r)
    assert np.array_equal(to_host(out.alpha), alpha_r)


# (5, 8192, 64, 4) exceeds the LDS-resident form and takes the global-list kernel; n > 64 takes
# two experts per lane (96: a partial second half)
@pytest.mark.parametrize("iters,m,n,k,seed", [(20, 4096, 64, 4, 0), (5, 4096, 64, 4, 0), (5, 4096, 64, 4, 1),
                                              (5, 4096, 64, 4, 2), (0, 512, 16, 2, 0), (3, 12, 4, 2, 0),
                                              (5, 8192, 64, 4, 0), (5, 2048, 128, 4, 0), (3, 1536, 96, 2, 0),
                                              (2, 2048, 128, 8, 0)])
def test_exact_completion_is_lp_optimum(iters, m, n, k, seed):
    spec = W.BalancedSpec(m=m, n=n, k=k)
    s = W.balanced_scores(spec, seed)
    say(f"[qb] exact m={m} n={n} k={k} iters={iters} seed={seed}")
    beta = torch.zeros(n, dtype=torch.float32, device=DEV)
    out = M.balance_duals(to_dev(s), k, beta, iters=iters, exact=True)
    torch.cuda.synchronize()
    _, beta_qb, _ = OB.qb_solve(s, k, iters)
    comp = OB.ssp_complete(s, k, beta_qb)
    gx = OB.idx_to_x(to_host(out.idx), n)
    assert np.array_equal(gx, comp.x), "GPU completion differs from the oracle's LP optimum"
    assert np.all(to_host(out.counts) == spec.q)
    info = to_host(out.info)
    assert info[2] == 1 and info[1] == comp.augmentations
    gb = to_host(beta).astype(np.float64)
    assert np.array_equal(to_host(beta), comp.beta.astype(np.float32))
    primal = OB.objective(s, gx)
    dual = OB.dual_objective(s, OB.best_alpha(s, gb, k), gb, k)
    assert dual == pytest.approx(primal, rel=1e-6)
    if m * n <= 64:
        cnt, best = OB.brute_force_dp(s, k)
        assert primal == pytest.approx(best, abs=1e-9)


# ------------------------------------------------------------------ stats
def test_stats_bias_and_global_accumulation():
    n, k, m = 256, 8, 4096
    rng = np.random.default_rng(0)
    counts = rng.multinomial(m * k, rng.dirichlet(np.ones(n) * 2)).astype(np.int32)
    counts[:3] = m * k // n                       # a few exactly balanced experts
    psum = (rng.random(n) * 40).astype(np.float32)
    bias0 = (rng.integers(-3, 4, n) * np.float32(1e-3)).astype(np.float32)
    gcounts0 = rng.integers(0, 10 ** 6, n).astype(np.int64)
    bias = to_dev(bias0)
    gc = to_dev(gcounts0)
    gt = to_dev(np.array([123456], np.int64))
    st = M.stats(m, k, to_dev(counts), to_dev(psum), alpha=1e-2, global_counts=gc, global_tokens=gt, bias=bias,
                 gamma=1e-3)
    torch.cuda.synchronize()
    f, P, aux = OS.switch_stats(counts, psum.astype(np.float64), m, 1e-2)
    assert np.array_equal(to_host(st.f), f.astype(np.float32))      # m is a power of two
    assert_rel(to_host(st.P), P, 1e-6, "P")
    assert_rel(to_host(st.aux), [aux], 1e-5, "aux")
    assert np.array_equal(to_host(bias), OS.lossfree_update(bias0, counts, m, k, 1e-3))
    assert np.array_equal(to_host(gc), gcounts0 + counts)
    assert to_host(gt)[0] == 123456 + m


def test_global_aux():
    n, nb = 128, 16
    rng = np.random.default_rng(1)
    gb = OS.GlobalBatch(n)
    P_rows = []
    for t in range(nb):
        c = rng.multinomial(4096, rng.dirichlet(np.ones(n)))
        ps = rng.dirichlet(np.ones(n)) * 4096
        gb.add(c, 4096, ps)
        P_rows.append((ps / 4096).astype(np.float32))
    P_rows = np.stack(P_rows)
    gb.prob_means = [p.astype(np.float64) for p in P_rows]
    fg, losses, mean = M.global_aux(to_dev(gb.counts), to_dev(np.array([gb.tokens], np.int64)), to_dev(P_rows))
    torch.cuda.synchronize()
    assert_rel(to_host(fg), gb.f(), 1e-7, "global f")
    assert_rel(to_host(losses), gb.losses(1e-2), 1e-5, "per-micro-batch losses")
    assert_rel(to_host(mean), [gb.loss(1e-2)], 1e-5, "global loss")


def test_global_aux_hybrid():
    # the global-batch loss plus 0.01 times each micro-batch's own Switch loss, the micro-batch
    # losses taken from moe_stats on the GPU (counts and score sums of each micro-batch)
    n, nb, m = 64, 8, 2048
    rng = np.random.default_rng(2)
    gb = OS.GlobalBatch(n)
    micro_gpu, P_rows = [], []
    for t in range(nb):
        c = rng.multinomial(m, rng.dirichlet(np.full(n, 0.5))).astype(np.int32)
        ps = (rng.dirichlet(np.ones(n)) * m).astype(np.float32)
        gb.add(c, m, ps.astype(np.float64))
        st = M.stats(m, 1, to_dev(c), to_dev(ps), alpha=1e-2)
        micro_gpu.append(st.aux)
        P_rows.append(to_host(st.P))
    P_rows = np.stack(P_rows)
    gb.prob_means = [p.astype(np.float64) for p in P_rows]   # the P rows the kernel sees (fp32)
    micro = torch.cat(micro_gpu)
    assert_rel(to_host(micro), gb.micro_losses(1e-2), 1e-5, "micro-batch losses (moe_stats)")
    # both readings of the page's constant weight 0.01: on the micro-batch loss, or on the global one
    for wg, wm in ((1.0, 1e-2), (1e-2, 1.0)):
        losses, hybrid, hmean = M.global_aux_hybrid(to_dev(gb.counts), to_dev(np.array([gb.tokens], np.int64)),
                                                    to_dev(P_rows), micro, alpha=1e-2, global_weight=wg,
                                                    micro_weight=wm)
        torch.cuda.synchronize()
        assert_rel(to_host(losses), gb.losses(1e-2), 1e-5, "global losses")
        assert_rel(to_host(hybrid), gb.hybrid_losses(1e-2, wg, wm), 1e-5, f"hybrid losses ({wg}, {wm})")
        assert_rel(to_host(hmean), [gb.hybrid_loss(1e-2, wg, wm)], 1e-5, f"hybrid mean ({wg}, {wm})")


# ------------------------------------------------------------------ whole layer
def _layer_check(spec, seed, cf, ffn, k=1):
    inp = W.switch_inputs(spec, seed)
    cap = OD.capacity(spec.T, spec.N, cf)
    w1 = w2 = None
    if ffn:
        w1, w2 = W.all_expert_weights(spec, seed)
    say(f"[layer] {spec.name} T={spec.T} k={k} cf={cf} cap={cap} ffn={ffn}")
    o = M.switch_layer(to_dev(inp.x), to_dev(inp.w_r), k=k, capacity=cap, alpha=spec.alpha,
                       w1=None if w1 is None else to_dev(w1), w2=None if w2 is None else to_dev(w2))
    torch.cuda.synchronize()
    ref = OR.route(inp.x, inp.w_r, k)
    idx = to_host(o.idx)
    flips = check_selection(idx, ref, f"{spec.name} layer")
    f, P, aux = OS.switch_stats(ref.counts, ref.prob_sum, spec.T, spec.alpha)
    assert_rel(to_host(o.P), P, 1e-5, "P")
    assert_rel(to_host(o.aux), [aux], 1e-5, "aux")
    # Downstream stages are checked against the oracle run on the GPU's selection: it equals the
    # oracle's own except on near-tie tokens (just checked), whose flips must not cascade.  The gate
    # of a chosen expert is the oracle's score of that expert.
    sel = idx.astype(np.int64)
    gate_sel = np.take_along_axis(ref.probs, sel, axis=1)
    counts_sel = np.bincount(sel.ravel(), minlength=spec.N)
    if not flips:
        assert np.array_equal(sel, ref.idx) and np.array_equal(counts_sel, ref.counts)
    assert np.array_equal(to_host(o.counts), counts_sel)
    assert np.array_equal(to_host(o.f), (counts_sel / spec.T).astype(np.float32))
    dm = OD.dispatch_maps(sel, spec.N, cap, padded=True)   # the layer's layout with a capacity
    assert np.array_equal(to_host(o.token_to_row), dm.token_to_row)
    assert np.array_equal(to_host(o.drop_mask), dm.drop_mask)
    assert np.array_equal(to_host(o.expert_offsets), dm.expert_offsets)
    assert np.array_equal(to_host(o.expert_rows), dm.expert_rows)
    filled = dm.filled_rows()
    assert np.array_equal(to_host(o.row_to_token)[filled], dm.row_to_token[filled])
    assert np.array_equal(to_host(o.dispatched)[filled], OD.dispatch_rows(inp.x, dm)[filled])
    x64 = OR.decode_hidden(inp.x)
    Y = np.zeros((dm.rows, spec.d))
    D64 = x64[dm.row_to_token[filled]]
    if ffn:
        for e in range(spec.N):
            lo, hi = dm.expert_offsets[e], dm.expert_offsets[e] + dm.expert_rows[e]
            if hi > lo:
                Y[lo:hi] = OE.relu_ffn(x64[dm.row_to_token[lo:hi]], w1[e], w2[e])
        tol = 2e-2
    else:
        Y[filled] = D64
        tol = 1e-5 if spec.x_dtype == "f32" else 2.0 ** -8 + 1e-5
    out_ref = OE.combine(x64, Y, gate_sel, dm.token_to_row)
    got = OR.decode_hidden(to_host(o.out))
    err = row_rel_err(got, out_ref)
    say(f"[layer] worst row error {err.max():.3e} (tol {tol:.1e}); near-tie flips {len(flips)}")
    assert err.max() <= tol
    dropped = np.all(dm.drop_mask == 1, axis=1)
    assert np.array_equal(to_host(o.out)[dropped], inp.x[dropped])
    return o


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_switch_layer(seed):
    _layer_check(W.TINY_SWITCH, seed, 1.25, ffn=False)


@pytest.mark.parametrize("cf,seed", [(1.0, 0), (1.25, 0), (1.25, 1), (1.25, 2)])
def test_switch_base_layer_with_ffn(cf, seed):
    _layer_check(W.SWITCH_BASE, seed, cf, ffn=True)


def test_switch_base_layer_identity_ragged():
    _layer_check(W.SWITCH_BASE.scaled(T=1234, d_ff=None), 1, 1.25, ffn=False)


@pytest.mark.parametrize("T,n,k,cf", [(5000, 200, 2, 1.1), (20000, 256, 1, 1.25)])
def test_layer_uneven_slices(T, n, k, cf):
    # the dispatch spreads each expert's slot-base sources over 1024 / n threads: n = 200 leaves
    # threads idle, and T = 20000 (625 chunks, 40 per super chunk) at n = 256 has more sources per
    # thread than its first batch of loads holds
    spec = W.SwitchSpec("uneven", T=T, d=128, N=n, w_r_std=0.05)
    _layer_check(spec, 5, cf, ffn=False, k=k)


def test_layer_large_batch():
    _layer_check(W.SWITCH_BASE.scaled(T=12000, d_ff=None), 2, 1.0, ffn=False)


@pytest.mark.parametrize("T,cf", [(2048, 1.0), (333, 1.5)])
def test_top2_layer(T, cf):
    spec = W.SwitchSpec("top2", T=T, d=256, N=64, w_r_std=0.05)
    _layer_check(spec, 3, cf, ffn=False, k=2)


def test_layer_maps_equal_separate_calls():
    # the layer (route kernel that also finishes the capacity prefix) against route + dispatch as separate calls
    spec = W.SWITCH_BASE.scaled(T=4000, d_ff=None)
    inp = W.switch_inputs(spec, 4)
    cap = OD.capacity(spec.T, spec.N, 1.0)
    x, w = to_dev(inp.x), to_dev(inp.w_r)
    o = M.switch_layer(x, w, k=1, capacity=cap)
    r = M.route(x, w, 1)
    dsp = M.dispatch(x, r.idx, spec.N, cap)
    torch.cuda.synchronize()
    assert torch.equal(o.idx, r.idx)
    assert torch.equal(o.token_to_row, dsp.token_to_row)
    assert torch.equal(o.drop_mask, dsp.drop_mask)
    assert torch.equal(o.expert_offsets, dsp.expert_offsets)
    assert torch.equal(o.expert_rows, dsp.expert_rows)
    assert torch.equal(o.row_to_token, dsp.row_to_token)
    filled = dsp.row_to_token >= 0
    assert torch.equal(o.dispatched[filled], dsp.dispatched[filled])
    # a second layer call on the same workspace: the control words were left zero
    o2 = M.switch_layer(x, w, k=1, capacity=cap)
    torch.cuda.synchronize()
    assert torch.equal(o2.token_to_row, o.token_to_row) and torch.equal(o2.dispatched[filled], o.dispatched[filled])


def _lossfree_step(spec, x_dev, w_dev, bias, gc, gt, fused):
    """One Loss-Free micro-batch: the single fused call, or route followed by moe_stats."""
    if fused:
        return M.route_lossfree(x_dev, w_dev, spec.k, bias, spec.gamma, global_counts=gc, global_tokens=gt)
    r = M.route(x_dev, w_dev, spec.k, score="sigmoid", bias=bias)
    M.stats(spec.T, spec.k, r.counts, r.prob_sum, global_counts=gc, global_tokens=gt, bias=bias, gamma=spec.gamma)
    return r


def _lossfree_loop(spec, inp, batches, bias, gc, gt, b_in=None, fused=False):
    """Route micro-batches [batches] with the running bias on the GPU, each followed by the bias
    update and global counts (moe_stats, or in the same launch with fused=True).  Each micro-batch
    is checked against the oracle routed with the bias the GPU held before it (so a near-tie flip
    in one micro-batch cannot cascade), and the GPU's bias update against the oracle's update from
    the GPU's counts.  Returns the number of near-tie flips."""
    w_dev = to_dev(inp.w_r)
    b_prev = to_host(bias).copy() if b_in is None else b_in
    nflips = 0
    for t in batches:
        x = inp.micro_batch(t)
        r = _lossfree_step(spec, to_dev(x), w_dev, bias, gc, gt, fused)
        torch.cuda.synchronize()
        ref = OR.route(x, inp.w_r, spec.k, score="sigmoid", bias=b_prev)
        gidx = to_host(r.idx)
        flips = check_selection(gidx, ref, f"micro-batch {t}")
        nflips += len(flips)
        gcounts = to_host(r.counts)
        assert np.array_equal(gcounts, np.bincount(gidx.ravel(), minlength=spec.N))
        if not flips:
            assert np.array_equal(gcounts, ref.counts)
        b_gpu = to_host(bias)
        assert np.array_equal(b_gpu, OS.lossfree_update(b_prev, gcounts, spec.T, spec.k, spec.gamma))
        b_prev = b_gpu
        vio = OS.load_violation(gcounts)
        say(f"  micro-batch {t}: MaxVio {vio[0]:.3f} near-tie flips {len(flips)}")
    return nflips


@pytest.mark.parametrize("fused,seed", [(False, 0), (True, 0), (True, 1), (True, 2)])
def test_lossfree_micro_batch_loop(fused, seed):
    """16 micro-batches: route with the old bias, accumulate global counts, then update the
    bias (route + moe_stats, or moe_route_lossfree alone).  Without near-tie flips the GPU's bias
    chain and global counts equal the oracle's own chain; with them, each step is still checked
    on the GPU's inputs (stage isolation)."""
    spec = W.LOSSFREE
    inp = W.lossfree_inputs(spec, seed)
    say(f"[lossfree] 16 micro-batches fused={fused} seed={seed}")
    bias = torch.zeros(spec.N, dtype=torch.float32, device=DEV)
    gc = torch.zeros(spec.N, dtype=torch.int64, device=DEV)
    gt = torch.zeros(1, dtype=torch.int64, device=DEV)
    nflips = _lossfree_loop(spec, inp, range(spec.micro_batches), bias, gc, gt, fused=fused)
    assert to_host(gt)[0] == spec.T * spec.micro_batches
    assert to_host(gc).sum() == spec.T * spec.k * spec.micro_batches
    if nflips == 0:   # the pure oracle chain, start to end
        b_ref = np.zeros(spec.N, np.float32)
        gb = OS.GlobalBatch(spec.N)
        for t in range(spec.micro_batches):
            ref = OR.route(inp.micro_batch(t), inp.w_r, spec.k, score="sigmoid", bias=b_ref)
            gb.add(ref.counts, spec.T)
            b_ref = OS.lossfree_update(b_ref, ref.counts, spec.T, spec.k, spec.gamma)
        assert np.array_equal(to_host(bias), b_ref)
        assert np.array_equal(to_host(gc), gb.counts)


@pytest.mark.parametrize("T,d,N,k,globals_", [(4096, 2048, 256, 8, True), (1000, 256, 64, 6, True),
                                               (777, 128, 512, 8, True), (4096, 2048, 256, 8, False)])
def test_route_lossfree_equals_route_then_stats(T, d, N, k, globals_):
    """moe_route_lossfree does in the route's last workgroup what moe_stats does after it: over
    12 micro-batches the two chains agree bit for bit in picks, gates, counts, expert
    probability sums, bias and global counts.  N=512 takes the row kernel's finish instead of
    the fused kernel's."""
    spec = W.LOSSFREE.scaled(T=T, d=d, N=N, k=k, w_r_std=0.1 / np.sqrt(d))
    inp = W.lossfree_inputs(spec, 2)
    w_dev = to_dev(inp.w_r)
    say(f"[lossfree] fused vs route+stats T={T} d={d} N={N} k={k} globals={globals_}")
    state = []
    for _ in range(2):
        b = torch.zeros(N, dtype=torch.float32, device=DEV)
        g = torch.zeros(N, dtype=torch.int64, device=DEV) if globals_ else None
        t = torch.zeros(1, dtype=torch.int64, device=DEV) if globals_ else None
        state.append((b, g, t))
    for step in range(12):
        x = to_dev(inp.micro_batch(step))
        r0 = _lossfree_step(spec, x, w_dev, *state[0], fused=False)
        r1 = _lossfree_step(spec, x, w_dev, *state[1], fused=True)
        torch.cuda.synchronize()
        for name in ("idx", "gate", "counts", "prob_sum"):
            assert torch.equal(getattr(r0, name), getattr(r1, name)), f"step {step}: {name}"
        assert torch.equal(state[0][0], state[1][0]), f"step {step}: bias"
        if globals_:
            assert torch.equal(state[0][1], state[1][1]) and torch.equal(state[0][2], state[1][2])
    assert float(state[1][0].abs().max()) > 0          # the bias moved
    if globals_:
        assert int(state[1][2][0]) == 12 * T and int(state[1][1].sum()) == 12 * T * k


@pytest.mark.parametrize("m,d,n,k,cf", [(4096, 256, 64, 4, 1.25), (2048, 128, 512, 4, 1.25), (1000, 128, 512, 32, -1)])
def test_switch_layer_lossfree_update(m, d, n, k, cf):
    """moe_switch_layer with the Loss-Free update (bias, global counts and tokens) equals the
    layer routed with the same bias followed by moe_stats, bit for bit, over 3 micro-batches:
    n = 64 has the dispatch derive the statistics, n = 512 (k = 4) the route's finish with the
    capacity prefix, n = 512 (k = 32) the route's finish before a separate dispatch histogram.
    Each update also equals the oracle's from the GPU's counts."""
    spec = W.LOSSFREE.scaled(T=m, d=d, N=n, k=k, w_r_std=0.1 / np.sqrt(d))
    inp = W.lossfree_inputs(spec, 3)
    w_dev = to_dev(inp.w_r)
    cap = int(cf * m * k / n) if cf > 0 else -1
    say(f"[lossfree] layer update m={m} d={d} n={n} k={k} capacity={cap}")
    st = [(torch.zeros(n, dtype=torch.float32, device=DEV), torch.zeros(n, dtype=torch.int64, device=DEV),
           torch.zeros(1, dtype=torch.int64, device=DEV)) for _ in range(2)]
    for step in range(3):
        x = to_dev(inp.micro_batch(step))
        b_prev = to_host(st[0][0]).copy()
        o1 = M.switch_layer(x, w_dev, k=k, capacity=cap, bias=st[0][0], score="sigmoid", update_bias=True,
                            gamma=spec.gamma, global_counts=st[0][1], global_tokens=st[0][2])
        o2 = M.switch_layer(x, w_dev, k=k, capacity=cap, bias=st[1][0], score="sigmoid")
        M.stats(m, k, o2.counts, o2.prob_sum, global_counts=st[1][1], global_tokens=st[1][2], bias=st[1][0],
                gamma=spec.gamma)
        torch.cuda.synchronize()
        for name in ("idx", "gate", "counts", "token_to_row", "out"):
            assert torch.equal(getattr(o1, name), getattr(o2, name)), f"step {step}: {name}"
        for u, v in zip(st[0], st[1]):
            assert torch.equal(u, v), f"step {step}: Loss-Free state"
        counts = to_host(o1.counts)
        assert np.array_equal(to_host(st[0][0]), OS.lossfree_update(b_prev, counts, m, k, spec.gamma))
    assert float(st[0][0].abs().max()) > 0
    assert int(st[0][2][0]) == 3 * m and int(st[0][1].sum()) == 3 * m * k


def test_lossfree_resume_is_bit_identical():
    """Checkpoint / resume: 16 micro-batches straight against 8, a host copy of the caller-owned
    state (bias, global counts, global tokens) restored into fresh buffers, then the other 8.
    The library keeps no state between calls, so the two runs agree bit for bit."""
    spec = W.LOSSFREE
    inp = W.lossfree_inputs(spec, 1)
    w_dev = to_dev(inp.w_r)

    def run(batches, bias, gc, gt):
        for t in batches:
            r = M.route(to_dev(inp.micro_batch(t)), w_dev, spec.k, score="sigmoid", bias=bias)
            M.stats(spec.T, spec.k, r.counts, r.prob_sum, global_counts=gc, global_tokens=gt, bias=bias,
                    gamma=spec.gamma)
        torch.cuda.synchronize()
        return r

    fresh = lambda: (torch.zeros(spec.N, dtype=torch.float32, device=DEV),  # noqa: E731
                     torch.zeros(spec.N, dtype=torch.int64, device=DEV), torch.zeros(1, dtype=torch.int64, device=DEV))
    b1, g1, t1 = fresh()
    r1 = run(range(16), b1, g1, t1)
    b2, g2, t2 = fresh()
    run(range(8), b2, g2, t2)
    ckpt = [to_host(v).copy() for v in (b2, g2, t2)]       # the checkpoint: a copy of the state
    del b2, g2, t2
    b3, g3, t3 = (to_dev(v) for v in ckpt)
    r3 = run(range(8, 16), b3, g3, t3)
    say("[lossfree] resume after 8 of 16 micro-batches")
    assert np.array_equal(to_host(b1), to_host(b3))
    assert np.array_equal(to_host(g1), to_host(g3)) and np.array_equal(to_host(t1), to_host(t3))
    assert np.array_equal(to_host(r1.idx), to_host(r3.idx))
    assert np.array_equal(to_host(r1.gate), to_host(r3.gate))
