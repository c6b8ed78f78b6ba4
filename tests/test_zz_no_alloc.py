"""moe_route_noalloc (the route on the library's static scratch, for callers that cannot
allocate) against moe_route (caller workspace): the same kernels, so every output must agree
bit for bit.  Two calls in a row, the second on a smaller input, for each case."""
import ctypes

import numpy as np
import pytest

import workloads as W
from load_balanced_expert_amd import _lib as L
from tests.gpu_util import DEV, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("load_balanced_expert_amd")


def _outputs(m, n, k):
    return (torch.empty((m, k), dtype=torch.int32, device=DEV), torch.empty((m, k), dtype=torch.float32, device=DEV),
            torch.empty(n, dtype=torch.int32, device=DEV), torch.empty(n, dtype=torch.float32, device=DEV))


def _noalloc(x, w, k, score, bias):
    """moe_route_noalloc through the C ABI with caller-allocated outputs."""
    m, d = x.shape
    n = w.shape[1]
    sh = M.shape(m, d, n, k, score, "prob", L.MOE_BF16 if x.dtype == torch.bfloat16 else L.MOE_F32)
    idx, g, c, ps = _outputs(m, n, k)
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    st = M.load().moe_route_noalloc(ctypes.byref(sh), p(x), p(w), None, p(bias), p(idx), p(g), p(c), p(ps),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.MOE_OK, f"moe_route_noalloc returned {st}"
    return idx, g, c, ps


CASES = [
    # (name, big spec, small T, k, score, with bias)
    ("switch-base", W.SWITCH_BASE, 3000, 1, "softmax", False),        # 256 tiles, then K split over 2 groups
    ("loss-free", W.LOSSFREE, 1000, 8, "sigmoid", True),              # K split, about 9 MB of scratch
    ("tiny fp32", W.TINY_SWITCH, 100, 1, "softmax", False),          # vector-ALU product
]


@pytest.mark.parametrize("name,spec,small,k,score,with_bias", CASES)
def test_route_noalloc_matches_route(name, spec, small, k, score, with_bias):
    inp = W.lossfree_inputs(spec, 0) if name == "loss-free" else W.switch_inputs(spec, 0)
    x_all = inp.micro_batch(0) if name == "loss-free" else inp.x
    w = to_dev(inp.w_r)
    bias = to_dev((np.random.default_rng(1).standard_normal(spec.N) * 1e-2).astype(np.float32)) if with_bias else None
    for T in (x_all.shape[0], small):   # two calls in a row, the second smaller
        say(f"[noalloc] {name} T={T} k={k} {score} bias={with_bias}")
        x = to_dev(x_all[:T])
        a = _noalloc(x, w, k, score, bias)
        r = M.route(x, w, k, score=score, bias=bias)
        torch.cuda.synchronize()
        for got, ref in zip(a, (r.idx, r.gate, r.counts, r.prob_sum)):
            assert np.array_equal(to_host(got), to_host(ref))
        assert int(to_host(a[2]).sum()) == T * k


def test_route_noalloc_rejects_too_large():
    # 65536 tokens x 2048 experts pass their logits through the scratch: 512 MiB, beyond 16 MiB
    sh = M.shape(65536, 1024, 2048, 1)
    f = ctypes.c_void_p(256)
    assert M.load().moe_route_noalloc(ctypes.byref(sh), f, f, None, None, f, f, f, None, None) == L.MOE_ERR_UNSUPPORTED
    assert M.load().moe_route_noalloc_max_bytes() == 16 << 20
