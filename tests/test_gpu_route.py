"""GPU parity: moe_route (router GEMM, scores, top-k, gates, counts, score sums)
against the float64 oracle on the same seeded inputs."""
import numpy as np
import pytest

import workloads as W
from oracle import router as OR
from tests.gpu_util import DEV, assert_rel, check_selection, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("load_balanced_expert_amd")


def run_route(x, w_r, k, score="softmax", gate="prob", bias=None):
    r = M.route(to_dev(x), to_dev(w_r), k, score=score, gate=gate,
                bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    return to_host(r.idx), to_host(r.gate), to_host(r.counts), to_host(r.prob_sum)


def check_route(x, w_r, k, what, score="softmax", gate="prob", bias=None):
    say(f"[route] {what}: m={x.shape[0]} d={x.shape[1]} n={w_r.shape[1]} k={k} {score} {gate} "
        f"bias={'yes' if bias is not None else 'no'}")
    idx, g, counts, psum = run_route(x, w_r, k, score, gate, bias)
    ref = OR.route(x, w_r, k, score=score, bias=bias, gate=gate)
    n = w_r.shape[1]
    assert idx.min() >= 0 and idx.max() < n
    flips = check_selection(idx, ref, what)
    same = np.array([t not in flips for t in range(x.shape[0])])
    assert_rel(g[same], ref.gate[same], 1e-5, f"{what} gates")
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=n)), f"{what}: counts != histogram of idx"
    if not flips:
        assert np.array_equal(counts, ref.counts)
    assert_rel(psum, ref.prob_sum, 1e-5, f"{what} prob_sum", floor=1e-6 * x.shape[0] / n)
    return idx, g, counts, psum, ref


def test_tiny_switch_fp32():
    inp = W.switch_inputs(W.TINY_SWITCH, 0)
    check_route(inp.x, inp.w_r, 1, "tiny switch (fp32 x, vector-ALU product)")


@pytest.mark.parametrize("seed", [0, 1])
def test_switch_base_ragged(seed):
    spec = W.SWITCH_BASE.scaled(T=1000)
    inp = W.switch_inputs(spec, seed)
    check_route(inp.x, inp.w_r, 1, "switch-base ragged T=1000 (bf16x3 MFMA)")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_switch_base_full(seed):
    inp = W.switch_inputs(W.SWITCH_BASE, seed)
    check_route(inp.x, inp.w_r, 1, "switch-base T=8192 d=768 N=128")


@pytest.mark.parametrize("T,d,n,k,score", [(1000, 800, 128, 1, "softmax"), (3000, 800, 128, 2, "softmax"),
                                          (2500, 2080, 256, 8, "sigmoid")])
def test_k_split_uneven_ranges(T, d, n, k, score):
    # few token tiles: each tile's K range is split over 2 or 4 workgroups; d / 32 K blocks that do
    # not divide evenly give ranges of two sizes, each staged in LDS at its own width
    spec = W.SwitchSpec("ksplit", T=T, d=d, N=n, w_r_std=0.1 / np.sqrt(d))
    inp = W.switch_inputs(spec, 7)
    bias = None
    if score == "sigmoid":
        bias = np.random.default_rng(7).normal(0.0, 0.01, n).astype(np.float32)
    check_route(inp.x, inp.w_r, k, f"K split, d={d} n={n} T={T}", score=score, bias=bias)


def test_padded_expert_count_and_odd_tokens():
    spec = W.SwitchSpec("odd", T=333, d=96, N=40, w_r_std=0.05)
    inp = W.switch_inputs(spec, 3)
    check_route(inp.x, inp.w_r, 3, "N=40 k=3 T=333")


def test_topk_renorm_gate():
    spec = W.SwitchSpec("renorm", T=512, d=128, N=64, w_r_std=0.05)
    inp = W.switch_inputs(spec, 4)
    check_route(inp.x, inp.w_r, 4, "top-4 renormalised softmax gate", gate="renorm")


def test_lossfree_micro_batch_with_bias():
    spec = W.LOSSFREE
    inp = W.lossfree_inputs(spec, 0)
    x = inp.micro_batch(1)
    g = np.random.default_rng(0)
    bias = (g.integers(-5, 6, spec.N) * np.float32(1e-3)).astype(np.float32)
    check_route(x, inp.w_r, spec.k, "loss-free micro-batch (sigmoid, top-8 of 256, bias)", score="sigmoid",
                bias=bias)


def test_sigmoid_without_bias():
    spec = W.LOSSFREE.scaled(T=700, d=256)
    inp = W.lossfree_inputs(spec, 1)
    check_route(inp.micro_batch(0), inp.w_r, 8, "sigmoid top-8 no bias T=700", score="sigmoid")


def test_softmax_with_bias():
    spec = W.SwitchSpec("sbias", T=256, d=64, N=32, w_r_std=0.2)
    inp = W.switch_inputs(spec, 5)
    bias = np.linspace(-0.02, 0.02, 32).astype(np.float32)
    check_route(inp.x, inp.w_r, 2, "softmax + bias (key = p + b)", bias=bias)


@pytest.mark.parametrize("k,score,bias", [(32, "softmax", False), (40, "softmax", False), (33, "sigmoid", True),
                                          (64, "softmax", True)])
def test_many_picks(k, score, bias):
    # k = 32 is the largest pick count of the half-wave epilogue; larger k takes the wave-per-token one
    spec = W.SwitchSpec("manyk", T=300, d=64, N=64, w_r_std=0.1)
    inp = W.switch_inputs(spec, 12)
    b = np.linspace(-0.01, 0.01, 64).astype(np.float32)[::-1].copy() if bias else None
    check_route(inp.x, inp.w_r, k, f"top-{k} of 64 ({score})", score=score, gate="renorm", bias=b)


@pytest.mark.parametrize("n,k", [(96, 1), (96, 3), (200, 2), (160, 1)])
def test_expert_counts_between_tile_sizes(n, k):
    # n not in {32, 64, 128, 256}: padded to the next of them (prepared planes, masked columns)
    spec = W.SwitchSpec(f"n{n}", T=300, d=128, N=n, w_r_std=0.05)
    inp = W.switch_inputs(spec, 13)
    check_route(inp.x, inp.w_r, k, f"N={n} top-{k}")


def test_fp32_x_fused_many_experts():
    # vector-ALU product with more experts than one lane group: four experts per lane in the epilogue
    spec = W.SwitchSpec("f32n100", T=150, d=40, N=100, x_dtype="f32", w_r_std=0.05)
    inp = W.switch_inputs(spec, 14)
    check_route(inp.x, inp.w_r, 3, "fp32 x, N=100 top-3 (vector-ALU product)")


def test_top1_renorm_gate_is_one():
    spec = W.SwitchSpec("renorm1", T=200, d=64, N=64, w_r_std=0.1)
    inp = W.switch_inputs(spec, 15)
    _, g, *_ = check_route(inp.x, inp.w_r, 1, "top-1 renormalised gate", gate="renorm")
    assert np.all(g == 1.0)


def test_bf16_x_with_d_not_multiple_of_8():
    spec = W.SwitchSpec("oddd", T=200, d=36, N=16, w_r_std=0.1)
    inp = W.switch_inputs(spec, 6)
    check_route(inp.x, inp.w_r, 2, "bf16 x, d=36 (vector-ALU product)")


def test_large_expert_count_path():
    spec = W.SwitchSpec("bign", T=777, d=256, N=600, w_r_std=0.05)
    inp = W.switch_inputs(spec, 7)
    check_route(inp.x, inp.w_r, 2, "N=600 (logits GEMM + row kernel)")


@pytest.mark.parametrize("T,d,n,gate", [(1000, 256, 1000, "prob"), (700, 128, 3000, "prob"), (530, 96, 520, "renorm")])
def test_large_expert_count_top1(T, d, n, gate):
    # top-1 softmax without bias on the big-n path: LDS sub-tiles of 32768 / npad tokens (10 at
    # n = 3000, so the last sub-tile of a workgroup is short), padded experts masked in the tile
    spec = W.SwitchSpec("bign1", T=T, d=d, N=n, w_r_std=0.05)
    inp = W.switch_inputs(spec, 9)
    check_route(inp.x, inp.w_r, 1, f"N={n} top-1 (logits GEMM + row kernel)", gate=gate)


def test_large_expert_count_fp32():
    spec = W.SwitchSpec("bignf", T=100, d=40, N=300, x_dtype="f32", w_r_std=0.05)
    inp = W.switch_inputs(spec, 8)
    check_route(inp.x, inp.w_r, 1, "N=300 fp32 x (vector-ALU logits)")


def test_ties_go_to_lower_index():
    # duplicated router columns: every token sees equal logits for experts 2j and 2j+1
    spec = W.SwitchSpec("ties", T=256, d=64, N=16, w_r_std=0.1)
    inp = W.switch_inputs(spec, 9)
    w = inp.w_r.copy()
    w[:, 1::2] = w[:, 0::2]
    idx, g, counts, _, ref = check_route(inp.x, w, 2, "exact ties")
    assert np.all(idx[:, 0] % 2 == 0) and np.all(idx[:, 1] == idx[:, 0] + 1)


def test_zero_router_uniform():
    x = W.switch_inputs(W.TINY_SWITCH.scaled(x_dtype="bf16"), 0).x
    idx, g, counts, psum = run_route(x, np.zeros((64, 8), np.float32), 1)
    assert np.all(idx == 0) and np.all(g == np.float32(1 / 8))
    assert counts.tolist() == [1024, 0, 0, 0, 0, 0, 0, 0]
    assert np.all(psum == np.float32(1024 / 8))


def test_repeat_is_bitwise_deterministic():
    inp = W.switch_inputs(W.SWITCH_BASE.scaled(T=2048), 11)
    a = run_route(inp.x, inp.w_r, 1)
    b = run_route(inp.x, inp.w_r, 1)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_switch_c_full_size(seed):
    """T=65536, d=1024, N=2048 at full size: the oracle routes every token (in blocks of 8192),
    so indices are checked on all tokens, gates on all but near-tie flips, counts against the
    oracle's and score sums against its full sums."""
    spec = W.SWITCH_C
    inp = W.switch_inputs(spec, seed)
    say(f"[route] switch-C full size on GPU, seed {seed}")
    idx, g, counts, psum = run_route(inp.x, inp.w_r, 1)
    psum_ref = np.zeros(spec.N)
    counts_ref = np.zeros(spec.N, np.int64)
    nflips = 0
    for lo in range(0, spec.T, 8192):
        ref = OR.route(inp.x[lo:lo + 8192], inp.w_r, 1)
        flips = check_selection(idx[lo:lo + 8192], ref, f"switch-C tokens {lo}..{lo + 8191}")
        nflips += len(flips)
        same = np.array([t not in flips for t in range(8192)])
        assert_rel(g[lo:lo + 8192][same], ref.gate[same], 1e-5, "switch-C gates")
        psum_ref += ref.prob_sum
        counts_ref += ref.counts
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=spec.N))
    if nflips == 0:
        assert np.array_equal(counts, counts_ref)
    assert_rel(psum, psum_ref, 1e-5, "switch-C prob_sum")


@pytest.mark.parametrize("n,k,score,bias,d", [(128, 1, "softmax", False, 768), (256, 8, "sigmoid", True, 256),
                                              (64, 40, "softmax", False, 64), (600, 1, "softmax", False, 128),
                                              (600, 3, "softmax", False, 128)])
def test_nan_rows_keep_indices_in_range(n, k, score, bias, d):
    # NaN inputs are outside the numerical contract, but indices stay in [0, n): NaN ranks as -inf,
    # so a row whose logits are all NaN picks experts 0..k-1; every other row routes as it does
    # without the NaN rows (tokens are routed independently), and counts follow the indices
    spec = W.SwitchSpec("nanrows", T=300, d=d, N=n, w_r_std=0.05)
    inp = W.switch_inputs(spec, 21)
    b = (np.random.default_rng(3).standard_normal(n) * 0.01).astype(np.float32) if bias else None
    say(f"[route] NaN rows: n={n} k={k} {score} bias={'yes' if bias else 'no'} d={d}")
    clean = run_route(inp.x, inp.w_r, k, score=score, bias=b)
    x = inp.x.copy()
    nan_rows = [0, 5, 31, 32, 299]
    x[nan_rows] = np.uint16(0x7FC0)   # bf16 quiet NaN
    idx, _, counts, _ = run_route(x, inp.w_r, k, score=score, bias=b)
    assert idx.min() >= 0 and idx.max() < n
    keep = np.setdiff1d(np.arange(spec.T), nan_rows)
    assert np.array_equal(idx[keep], clean[0][keep])
    assert np.all(idx[nan_rows] == np.arange(k)[None, :])
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=n))
