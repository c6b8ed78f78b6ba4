"""GPU parity: moe_dispatch (slots, drop mask, permutation maps, dispatched rows),
moe_combine and moe_expert_ffn, each fed the same generated inputs as the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import dispatch as OD
from oracle import expert as OE
from oracle import router as OR
from tests.gpu_util import DEV, assert_rel, row_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("load_balanced_expert_amd")

BF16_ROUND = 2.0 ** -8 + 1e-5     # one bf16 rounding of an fp32-accurate result, per-row relative


def check_dispatch(T, n, k, d, cf, skew, seed, x_dtype="bf16", copy_rows=True):
    idx = W.random_assignment(T, n, k, seed, skew)
    cap = -1 if cf is None else OD.capacity(T * k if k > 1 else T, n, cf)
    say(f"[dispatch] T={T} n={n} k={k} d={d} cap={cap} skew={skew} {x_dtype}")
    xs = W.switch_inputs(W.SwitchSpec("d", T=T, d=d, N=n, x_dtype=x_dtype), seed).x
    out = M.dispatch(to_dev(xs), to_dev(idx), n, capacity=cap, copy_rows=copy_rows)
    torch.cuda.synchronize()
    # capacity-padded layout with a capacity, compact without
    ref = OD.dispatch_maps(idx, n, cap if cap >= 0 else T * k, padded=cap >= 0)
    assert np.array_equal(to_host(out.token_to_row), ref.token_to_row)
    assert np.array_equal(to_host(out.drop_mask), ref.drop_mask)
    assert np.array_equal(to_host(out.expert_offsets), ref.expert_offsets)
    assert np.array_equal(to_host(out.expert_rows), ref.expert_rows)
    rows = ref.rows
    assert np.array_equal(to_host(out.row_to_token)[:rows], ref.row_to_token)
    if copy_rows:
        got = to_host(out.dispatched)[:rows]
        assert np.array_equal(got, OD.dispatch_rows(xs, ref)), "dispatched rows are not bit copies"
    return ref


@pytest.mark.parametrize("cf", [1.0, 1.25])
def test_switch_base_capacity(cf):
    ref = check_dispatch(8192, 128, 1, 768, cf, skew=1.0, seed=0)
    assert ref.drop_mask.sum() > 0


@pytest.mark.parametrize("T,n,k,d,cf,skew", [
    (1000, 16, 1, 64, 1.0, 1.5),       # ragged chunk, heavy overflow
    (3000, 7, 2, 40, 1.0, 0.5),        # k = 2, odd n, d % 8 != 0 rows
    (2500, 64, 4, 128, 0.75, 0.0),     # k = 4 (token-major slot priority)
    (513, 256, 8, 32, None, 0.3),      # unlimited capacity
    (4096, 2048, 1, 64, 1.25, 1.1),    # 2048 bins
    (70000, 128, 1, 16, 1.0, 0.8),     # many chunks
])
def test_dispatch_cases(T, n, k, d, cf, skew):
    check_dispatch(T, n, k, d, cf, skew, seed=1)


def test_dispatch_fp32_rows():
    check_dispatch(1024, 8, 1, 64, 1.25, 0.7, seed=2, x_dtype="f32")


def test_all_tokens_one_expert():
    T, n = 1000, 8
    idx = np.zeros((T, 1), np.int32)
    cap = OD.capacity(T, n, 1.25)
    out = M.dispatch(None, to_dev(idx), n, capacity=cap, d=16)
    torch.cuda.synchronize()
    assert int(to_host(out.drop_mask).sum()) == T - cap
    assert to_host(out.expert_offsets).tolist() == [j * cap for j in range(n + 1)]
    assert to_host(out.expert_rows).tolist() == [cap] + [0] * (n - 1)
    assert np.array_equal(to_host(out.token_to_row)[:cap, 0], np.arange(cap))


def test_switch_c_dispatch_full():
    check_dispatch(65536, 2048, 1, 1024, 1.25, skew=0.6, seed=3)


# ------------------------------------------------------------------ combine
def check_combine(T, n, k, d, cap, x_dtype, seed, residual=True):
    idx = W.random_assignment(T, n, k, seed, 0.8)
    dm = OD.dispatch_maps(idx, n, cap)
    rows = max(dm.rows, 1)
    y = W.random_rows(rows, d, seed, bf16=(x_dtype == "bf16"))
    gate = W.random_gates(T, k, seed)
    x = W.switch_inputs(W.SwitchSpec("c", T=T, d=d, N=n, x_dtype=x_dtype), seed).x
    say(f"[combine] T={T} k={k} d={d} rows={rows} {x_dtype} residual={residual}")
    out = M.combine(to_dev(y), to_dev(gate), to_dev(dm.token_to_row), to_dev(x) if residual else None,
                    out_dtype=torch.bfloat16 if x_dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    got = to_host(out)
    x64 = OR.decode_hidden(x)
    y64 = OR.decode_hidden(y)
    ref = OE.combine(x64, y64, gate, dm.token_to_row, residual=residual)
    g64 = OR.decode_hidden(got)
    tol = BF16_ROUND if x_dtype == "bf16" else 1e-5
    err = row_rel_err(g64, ref)
    assert err.max() <= tol, f"combine: worst row error {err.max():.3e}"
    dropped = np.all(dm.token_to_row < 0, axis=1)
    if residual and dropped.any():
        assert np.array_equal(got[dropped], x[dropped]), "dropped tokens must keep x bit-exactly"


@pytest.mark.parametrize("T,n,k,d,cap,xd", [(1024, 8, 1, 64, 160, "f32"), (8192, 128, 1, 768, 64, "bf16"),
                                            (999, 16, 2, 40, 100, "bf16"), (500, 32, 4, 64, 60, "f32")])
def test_combine(T, n, k, d, cap, xd):
    check_combine(T, n, k, d, cap, xd, seed=4)


def test_combine_without_residual():
    check_combine(512, 8, 2, 128, 100, "bf16", seed=5, residual=False)


def test_dispatch_capacity_zero():
    check_dispatch(300, 8, 2, 32, 0.0, 0.5, seed=8)


# ------------------------------------------------------------------ expert FFN
@pytest.mark.parametrize("rows_per_expert,d,d_ff", [([80, 37, 0, 130, 64, 1, 33, 96], 768, 3072),
                                                    ([5, 40, 17, 0], 1024, 4096), ([3, 200], 128, 96),
                                                    ([128, 129, 0, 256, 31], 256, 512)])
def test_expert_ffn(rows_per_expert, d, d_ff):
    n = len(rows_per_expert)
    spec = W.SwitchSpec("ffn", T=1, d=d, N=n, d_ff=d_ff, w_std=np.sqrt(1.0 / d))
    offs = np.zeros(n + 1, np.int32)
    offs[1:] = np.cumsum(rows_per_expert)
    rows = int(offs[-1])
    D = W.random_rows(rows, d, seed=6, bf16=True)
    w1, w2 = W.all_expert_weights(spec, 6)
    say(f"[ffn] n={n} d={d} d_ff={d_ff} rows={rows_per_expert}")
    y = M.expert_ffn(to_dev(D), to_dev(offs), to_dev(w1), to_dev(w2), rows_max=max(rows_per_expert))
    torch.cuda.synchronize()
    got = OR.decode_hidden(to_host(y))
    D64 = OR.decode_hidden(D)
    for e in range(n):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            continue
        ref = OE.relu_ffn(D64[lo:hi], w1[e], w2[e])
        err = row_rel_err(got[lo:hi], ref)
        assert err.max() <= 2e-2, f"expert {e}: worst row error {err.max():.3e}"


def test_expert_ffn_padded_layout():
    # capacity-padded rows: expert j's rows start at j * C, rows_j of them filled
    rows_per_expert, C, d, d_ff = [80, 0, 17, 80, 1, 64], 80, 256, 512
    n = len(rows_per_expert)
    spec = W.SwitchSpec("ffnp", T=1, d=d, N=n, d_ff=d_ff, w_std=np.sqrt(1.0 / d))
    offs = (np.arange(n + 1) * C).astype(np.int32)
    rows = np.array(rows_per_expert, np.int32)
    D = W.random_rows(n * C, d, seed=9, bf16=True)
    w1, w2 = W.all_expert_weights(spec, 9)
    say(f"[ffn padded] n={n} C={C} rows={rows_per_expert}")
    y = M.expert_ffn(to_dev(D), to_dev(offs), to_dev(w1), to_dev(w2), rows_max=C, expert_rows=to_dev(rows))
    torch.cuda.synchronize()
    got = OR.decode_hidden(to_host(y))
    D64 = OR.decode_hidden(D)
    for e in range(n):
        lo, hi = offs[e], offs[e] + rows[e]
        if hi == lo:
            continue
        ref = OE.relu_ffn(D64[lo:hi], w1[e], w2[e])
        err = row_rel_err(got[lo:hi], ref)
        assert err.max() <= 2e-2, f"expert {e}: worst row error {err.max():.3e}"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("T,d,n,k,d_ff,cf", [(8192, 768, 128, 1, 3072, 1.25), (1000, 256, 16, 2, 512, 1.25),
                                             (300, 512, 8, 1, 256, -1.0)])
def test_packed_expert_weights_bit_identical(T, d, n, k, d_ff, cf):
    # the FFN reading moe_expert_weights_pack's layout runs the same products in the same order as
    # the plain layout: every output of the layer is bit-identical
    spec = W.SwitchSpec("packed", T=T, d=d, N=n, d_ff=d_ff, w_std=np.sqrt(1.0 / d), w_r_std=0.1 / np.sqrt(d))
    inp = W.switch_inputs(spec, 5)
    w1, w2 = W.all_expert_weights(spec, 5)
    say(f"[ffn packed] T={T} d={d} n={n} k={k} d_ff={d_ff} cf={cf}")
    x, wr, W1, W2 = to_dev(inp.x), to_dev(inp.w_r), to_dev(w1), to_dev(w2)
    cap = M.capacity(T, n, cf) if cf > 0 else -1
    plain = M.switch_layer(x, wr, k=k, capacity=cap, w1=W1, w2=W2)
    P1, P2 = M.pack_expert_weights(W1), M.pack_expert_weights(W2)
    packed = M.switch_layer(x, wr, k=k, capacity=cap, w1=P1, w2=P2, weights_packed=True)
    torch.cuda.synchronize()
    assert not torch.equal(_bits(P1), _bits(W1))   # the layout did change
    for f in ("idx", "gate", "token_to_row", "expert_rows", "out"):
        assert torch.equal(_bits(getattr(plain, f)), _bits(getattr(packed, f))), f
    rows = plain.token_to_row.reshape(-1)
    kept = rows[rows >= 0].long()
    assert torch.equal(_bits(plain.y[kept]), _bits(packed.y[kept]))
    assert torch.equal(_bits(plain.hidden[kept]), _bits(packed.hidden[kept]))
