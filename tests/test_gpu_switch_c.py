"""GPU parity of the whole Switch layer at the Switch-C expert count: T=65536 tokens, d_model=1024,
N=2048 experts, top-1, capacity factor 1.25 (capacity 40), ReLU expert FFN d_ff=4096 with 34 GB of
bf16 expert weights on one GPU.

The expert weights are drawn on the GPU from a seeded torch generator (too large to draw on the
host in reasonable time); the slices of the sampled experts are copied to the host for the oracle.
Routing, statistics, capacity slots, drop mask, maps and every dispatched row are compared for all
tokens; expert outputs and combined rows for every token of a sample of experts that includes
experts past 1024 (their weights start beyond 2^31 elements of the stacked buffers)."""
import numpy as np
import pytest

import workloads as W
from oracle import dispatch as OD
from oracle import expert as OE
from oracle import router as OR
from oracle import stats as OS
from tests.gpu_util import DEV, assert_rel, check_selection, row_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("load_balanced_expert_amd")


def test_switch_c_layer_full_size():
    spec = W.SWITCH_C
    T, d, N, d_ff = spec.T, spec.d, spec.N, spec.d_ff
    inp = W.switch_inputs(spec, 0)
    cap = OD.capacity(T, N, 1.25)
    assert cap == 40
    say(f"[switch-C layer] T={T} d={d} N={N} d_ff={d_ff} cap={cap}: drawing 34 GB of expert weights")
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    W1 = torch.empty((N, d_ff, d), dtype=torch.bfloat16, device=DEV)
    W2 = torch.empty((N, d, d_ff), dtype=torch.bfloat16, device=DEV)
    for w in (W1, W2):
        for e0 in range(0, N, 256):
            w[e0:e0 + 256] = (torch.randn(w[e0:e0 + 256].shape, generator=g, device=DEV) * spec.w_std).to(
                torch.bfloat16)
    x_dev, w_dev = to_dev(inp.x), to_dev(inp.w_r)
    say("[switch-C layer] running moe_switch_layer")
    o = M.switch_layer(x_dev, w_dev, k=1, capacity=cap, alpha=spec.alpha, w1=W1, w2=W2)
    torch.cuda.synchronize()
    idx = to_host(o.idx)

    # routing on every token (oracle in blocks of 8192 tokens)
    say("[switch-C layer] oracle routing")
    probs_sel = np.zeros(T)
    psum_ref = np.zeros(N)
    counts_ref = np.zeros(N, np.int64)
    nflips = 0
    for lo in range(0, T, 8192):
        ref = OR.route(inp.x[lo:lo + 8192], inp.w_r, 1)
        nflips += len(check_selection(idx[lo:lo + 8192], ref, f"switch-C layer tokens {lo}.."))
        probs_sel[lo:lo + 8192] = np.take_along_axis(ref.probs, idx[lo:lo + 8192].astype(np.int64), axis=1)[:, 0]
        psum_ref += ref.prob_sum
        counts_ref += ref.counts
    # downstream stages on the GPU's selection (equal to the oracle's but for near-tie flips)
    counts_sel = np.bincount(idx.ravel(), minlength=N)
    if nflips == 0:
        assert np.array_equal(counts_sel, counts_ref)
    f, P, aux = OS.switch_stats(counts_sel, psum_ref, T, spec.alpha)
    assert np.array_equal(to_host(o.counts), counts_sel)
    assert np.array_equal(to_host(o.f), f.astype(np.float32))
    assert_rel(to_host(o.P), P, 1e-5, "P")
    assert_rel(to_host(o.aux), [OS.switch_stats(counts_ref, psum_ref, T, spec.alpha)[2]], 1e-5, "aux")
    assert_rel(to_host(o.gate)[:, 0], probs_sel, 1e-5, "gates")

    dm = OD.dispatch_maps(idx, N, cap, padded=True)
    assert np.array_equal(to_host(o.token_to_row), dm.token_to_row)
    assert np.array_equal(to_host(o.drop_mask), dm.drop_mask)
    assert np.array_equal(to_host(o.expert_offsets), dm.expert_offsets)
    assert np.array_equal(to_host(o.expert_rows), dm.expert_rows)
    filled = dm.filled_rows()
    say(f"[switch-C layer] {len(filled)} kept rows, {int(dm.drop_mask.sum())} drops, near-tie flips {nflips}")
    assert np.array_equal(to_host(o.row_to_token)[filled], dm.row_to_token[filled])
    assert np.array_equal(to_host(o.dispatched)[filled], inp.x[dm.row_to_token[filled]])

    # expert outputs and combined rows on a sample of experts, including the last ones
    rng = np.random.default_rng(5)
    sample = sorted(set([0, 1, 511, 512, 1023, 1024, 1025, 1535, 2046, 2047] +
                        rng.choice(N, 22, replace=False).tolist()))
    x64 = OR.decode_hidden(inp.x)
    y_gpu = o.y
    out_gpu = o.out
    worst_y = worst_out = 0.0
    checked = 0
    for e in sample:
        lo, n_e = int(dm.expert_offsets[e]), int(dm.expert_rows[e])
        if n_e == 0:
            continue
        toks = dm.row_to_token[lo:lo + n_e]
        w1 = to_host(W1[e]).copy()
        w2 = to_host(W2[e]).copy()
        Y = OE.relu_ffn(x64[toks], w1, w2)
        yg = OR.decode_hidden(to_host(y_gpu[lo:lo + n_e]))
        worst_y = max(worst_y, float(row_rel_err(yg, Y).max()))
        out_ref = x64[toks] + probs_sel[toks][:, None] * Y
        og = OR.decode_hidden(to_host(out_gpu[torch.as_tensor(toks, device=DEV)]))
        worst_out = max(worst_out, float(row_rel_err(og, out_ref).max()))
        checked += n_e
    say(f"[switch-C layer] {len(sample)} experts, {checked} rows: worst expert-output error {worst_y:.2e}, "
        f"worst combined-row error {worst_out:.2e}")
    assert checked > 0 and worst_y <= 2e-2 and worst_out <= 2e-2
    dropped = dm.drop_mask[:, 0] == 1
    assert np.array_equal(to_host(o.out)[dropped], inp.x[dropped])
    del W1, W2, o
    torch.cuda.empty_cache()
