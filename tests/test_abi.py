"""C-ABI contract of libmoe.so, checked on the host (no GPU needed).

Loads the library, checks that it exports every entry point declared in
include/moe.h, and that argument validation rejects bad calls before any
HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import load_balanced_expert_amd as M
from load_balanced_expert_amd import _lib as L
from oracle import dispatch as OD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from load_balanced_expert_amd import build
        build.build()
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"libmoe.so does not export {n}"
    assert set(names) == set(L.SIGNATURES), "binding signatures out of sync with include/moe.h"


def test_router_prepare_validation(lib):
    assert lib.moe_router_planes_bytes(768, 128) == 3 * 128 * 768 * 2
    assert lib.moe_router_planes_bytes(0, 128) == 0
    assert lib.moe_router_prepare(768, 128, None, FAKE, None) == 1
    assert lib.moe_router_prepare(768, 5000, FAKE, FAKE, None) == 2


def test_build_info(lib):
    assert b"gfx950" in lib.moe_build_info()


@pytest.mark.parametrize("m,n,cf", [(1024, 8, 1.25), (8192, 128, 1.0), (8192, 128, 1.25), (65536, 2048, 1.25),
                                    (10, 1, 0.3), (7, 3, 0.1), (1000, 7, 1.1), (16, 4, 2.0), (5, 5, 0.0),
                                    (123456, 37, 3.3333333)])
def test_capacity_matches_oracle(lib, m, n, cf):
    assert lib.moe_capacity(m, n, cf) == OD.capacity(m, n, cf)


def test_capacity_rejects_invalid(lib):
    assert lib.moe_capacity(-1, 4, 1.0) == -1
    assert lib.moe_capacity(10, 0, 1.0) == -1
    assert lib.moe_capacity(10, 4, -1.0) == -1
    assert lib.moe_capacity(10, 4, float("nan")) == -1
    assert lib.moe_capacity(10, 4, float("inf")) == -1
    assert lib.moe_capacity(2 ** 40, 1, 1.0) == -1      # exceeds int32


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_str(s)
    assert b"unknown" in lib.moe_status_str(99)


def _sh(m=64, d=32, n=8, k=1, score=0, gate=0, xd=1):
    return L.MoeShape(m, d, n, k, score, gate, xd)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("bad", [dict(m=0), dict(d=0), dict(n=0), dict(k=0), dict(k=9), dict(score=2),
                                 dict(gate=5), dict(xd=3)])
def test_invalid_shapes(lib, bad):
    sh = _sh(**bad)
    assert lib.moe_workspace_size(ctypes.byref(sh), -1, 0) == 0
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == L.MOE_ERR_INVALID_ARG


def test_unsupported_sizes(lib):
    sh = _sh(n=5000)
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == L.MOE_ERR_UNSUPPORTED
    sh = _sh(m=2 ** 31, k=1)
    assert lib.moe_workspace_size(ctypes.byref(sh), -1, 0) == 0
    sh = _sh(d=65537)
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == L.MOE_ERR_UNSUPPORTED
    sh = _sh(n=128, k=65)   # more picks per token than wave lanes
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == L.MOE_ERR_UNSUPPORTED


def test_null_pointers_rejected(lib):
    sh = _sh()
    assert lib.moe_route(ctypes.byref(sh), None, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.moe_dispatch(ctypes.byref(sh), -1, FAKE, None, FAKE, None, FAKE, None, None, None, FAKE, 1 << 30,
                            None) == 1
    assert lib.moe_dispatch(ctypes.byref(sh), -2, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, 1 << 30,
                            None) == 1
    # dispatched rows requested without x
    assert lib.moe_dispatch(ctypes.byref(sh), -1, None, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, 1 << 30,
                            None) == 1
    assert lib.moe_combine(ctypes.byref(sh), None, 1, FAKE, FAKE, None, FAKE, None) == 1
    assert lib.moe_combine(ctypes.byref(sh), FAKE, 7, FAKE, FAKE, None, FAKE, None) == 1


def test_route_lossfree_validation(lib):
    sh = _sh()
    big = 1 << 30
    ok = lambda **kw: dict(dict(x=FAKE, bias=FAKE, gamma=1e-3, gc=None, gt=None, ws=FAKE, wsb=big), **kw)  # noqa

    def call(a):
        return lib.moe_route_lossfree(ctypes.byref(sh), a["x"], FAKE, None, a["bias"], a["gamma"], FAKE, FAKE, FAKE,
                                      None, a["gc"], a["gt"], a["ws"], a["wsb"], None)

    assert call(ok(bias=None)) == L.MOE_ERR_INVALID_ARG          # the bias it updates is required
    assert call(ok(x=None)) == L.MOE_ERR_INVALID_ARG
    assert call(ok(gamma=float("nan"))) == L.MOE_ERR_INVALID_ARG
    assert call(ok(gamma=float("inf"))) == L.MOE_ERR_INVALID_ARG
    assert call(ok(gc=FAKE)) == L.MOE_ERR_INVALID_ARG            # global counts without global tokens
    assert call(ok(gt=FAKE)) == L.MOE_ERR_INVALID_ARG
    assert call(ok(wsb=1024)) == L.MOE_ERR_WORKSPACE
    assert call(ok(ws=None)) == L.MOE_ERR_INVALID_ARG
    bad = _sh(k=0)
    assert lib.moe_route_lossfree(ctypes.byref(bad), FAKE, FAKE, None, FAKE, 1e-3, FAKE, FAKE, FAKE, None, None,
                                  None, FAKE, big, None) == L.MOE_ERR_INVALID_ARG


def test_workspace_too_small_or_misaligned(lib):
    sh = _sh(m=1024, d=768, n=128)
    need = lib.moe_workspace_size(ctypes.byref(sh), -1, 0)
    assert need >= 4096 + 3 * 128 * 768 * 2     # control words + router weight planes
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, 1024, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, ctypes.c_void_p(0x1010),
                       1 << 40, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.moe_route(ctypes.byref(sh), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG


def test_workspace_grows_with_capacity_and_ffn(lib):
    sh = _sh(m=8192, d=768, n=128)
    a = lib.moe_workspace_size(ctypes.byref(sh), 64, 0)
    b = lib.moe_workspace_size(ctypes.byref(sh), 80, 0)
    c = lib.moe_workspace_size(ctypes.byref(sh), 80, 3072)
    assert 0 < a <= b < c
    assert lib.moe_workspace_size(ctypes.byref(sh), -2, 0) == 0


def test_stats_validation(lib):
    assert lib.moe_stats(0, 8, 1, FAKE, None, 0.01, None, None, None, None, None, None, 0.001, None) == 1
    assert lib.moe_stats(8, 8, 9, FAKE, None, 0.01, None, None, None, None, None, None, 0.001, None) == 1
    assert lib.moe_stats(8, 8, 1, None, None, 0.01, None, None, None, None, None, None, 0.001, None) == 1
    # global counts without global tokens
    assert lib.moe_stats(8, 8, 1, FAKE, None, 0.01, None, None, None, FAKE, None, None, 0.001, None) == 1
    # aux requested without prob_sum
    assert lib.moe_stats(8, 8, 1, FAKE, None, 0.01, None, None, FAKE, None, None, None, 0.001, None) == 1
    assert lib.moe_stats(8, 5000, 1, FAKE, None, 0.01, None, None, None, None, None, None, 0.001, None) == 2
    assert lib.moe_global_aux(8, None, FAKE, FAKE, 1, 0.01, None, None, None, None, 0.0, 0.0, None, None, None) == 1
    assert lib.moe_global_aux(8, FAKE, FAKE, None, 2, 0.01, None, None, None, None, 0.0, 0.0, None, None, None) == 1
    # a hybrid output needs the micro-batch losses
    assert lib.moe_global_aux(8, FAKE, FAKE, FAKE, 2, 0.01, None, None, None, None, 1.0, 0.01, FAKE, None, None) == 1


def test_balance_validation(lib):
    big = 1 << 40
    args = lambda m, n, k, it=1, mode=0, ex=0, ws=FAKE, wsb=big: (m, n, k, FAKE, FAKE, it, mode, ex, FAKE, FAKE,  # noqa
                                                                   None, None, ws, wsb, None)
    assert lib.moe_balance_duals(*args(10, 4, 1)) == 1          # (m*k) % n != 0
    assert lib.moe_balance_duals(*args(8, 4, 4)) == 1           # k == n
    assert lib.moe_balance_duals(*args(8, 4, 1, mode=2)) == 1
    assert lib.moe_balance_duals(*args(8, 4, 1, it=2, mode=1)) == 1   # online takes one step
    assert lib.moe_balance_duals(*args(8, 4, 1, mode=1, ex=1)) == 1   # exact is solve-only
    assert lib.moe_balance_duals(*args(256, 256, 1, ex=1)) == 2      # completion limited to n <= 128
    assert lib.moe_balance_duals(*args(1 << 16, 128, 2, ex=1)) == 2  # n > 64: the assignment must fit in LDS
    assert lib.moe_balance_duals(*args(64, 8, 1, wsb=100)) == 3
    assert lib.moe_balance_workspace_size(64, 8, 8, 0) == 0
    assert lib.moe_balance_workspace_size(4096, 64, 4, 1) > lib.moe_balance_workspace_size(4096, 64, 4, 0)


def test_expert_ffn_validation(lib):
    big = 1 << 40
    assert lib.moe_expert_ffn(8, 48, 64, 10, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == 2
    assert lib.moe_expert_ffn(8, 64, 64, 10, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == 1
    assert lib.moe_expert_ffn(8, 64, 64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == 3


def test_switch_layer_validation(lib):
    sh = _sh(m=64, d=64, n=8, xd=0)
    out = L.LayerOutputs()
    out.out = FAKE
    p = L.LayerParams(16, 1, 64, 0.01, None)                       # relu_ffn needs bf16 x
    assert lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None,
                                ctypes.byref(out), FAKE, 1 << 40, None) == 1
    p = L.LayerParams(16, 7, 0, 0.01, None)
    assert lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, None, None, None,
                                ctypes.byref(out), FAKE, 1 << 40, None) == 1
    out.out = None
    p = L.LayerParams(16, 0, 0, 0.01, None)
    assert lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, None, None, None,
                                ctypes.byref(out), FAKE, 1 << 40, None) == 1


def test_switch_layer_lossfree_validation(lib):
    sh = _sh(m=64, d=64, n=8, k=2, score=1, xd=0)
    out = L.LayerOutputs()
    out.out = FAKE
    other = ctypes.c_void_p(0x2000)

    def call(bias, **kw):
        p = L.LayerParams(16, 0, 0, 0.01, None)
        for key, v in kw.items():
            setattr(p, key, v)
        return lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, None, None, bias,
                                    ctypes.byref(out), FAKE, 1 << 40, None)

    assert call(FAKE, update_bias=other.value, gamma=1e-3) == L.MOE_ERR_INVALID_ARG   # not the routing bias
    assert call(None, update_bias=FAKE.value, gamma=1e-3) == L.MOE_ERR_INVALID_ARG
    assert call(FAKE, update_bias=FAKE.value, gamma=float("nan")) == L.MOE_ERR_INVALID_ARG
    assert call(FAKE, global_counts=FAKE.value) == L.MOE_ERR_INVALID_ARG               # without global tokens
    assert call(FAKE, global_tokens=FAKE.value) == L.MOE_ERR_INVALID_ARG
    assert call(FAKE, update_bias=FAKE.value, gamma=1e-3, global_counts=FAKE.value, global_tokens=None) == \
        L.MOE_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(M.MoeError):
        M.route(torch.zeros(4, 8), torch.zeros(8, 2), 1)


def test_signsgd_limits(lib):
    # more than 256 experts, or k >= n, are refused before any device work
    assert lib.moe_balance_signsgd(600, 300, 3, FAKE, FAKE, 0.01, 1, FAKE, FAKE, FAKE, 1 << 30, None) == \
        L.MOE_ERR_UNSUPPORTED
    assert lib.moe_balance_signsgd(64, 8, 8, FAKE, FAKE, 0.01, 1, FAKE, FAKE, FAKE, 1 << 30, None) == \
        L.MOE_ERR_INVALID_ARG
    assert lib.moe_balance_signsgd(64, 8, 2, FAKE, FAKE, -1.0, 1, FAKE, FAKE, FAKE, 1 << 30, None) == \
        L.MOE_ERR_INVALID_ARG


def test_minibatch_validation(lib):
    big = 1 << 40
    args = lambda m, n, k, br, it=1, mode=0, wsb=big: (m, n, k, FAKE, FAKE, it, mode, br, FAKE, FAKE,  # noqa
                                                       None, None, FAKE, wsb, None)
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 24)) == 1       # blocks do not tile the tokens
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 4)) == 1        # block quota 4·1/8 not whole
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 0)) == 1
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 16, it=2, mode=1)) == 1   # online takes one step
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 16, mode=3)) == 1
    assert lib.moe_balance_duals_minibatch(*args(64, 8, 1, 16, wsb=100)) == 3
    assert lib.moe_balance_minibatch_workspace_size(64, 8, 1, 24) == 0
    assert lib.moe_balance_minibatch_workspace_size(64, 8, 1, 16) > lib.moe_balance_workspace_size(64, 8, 1, 0)


def test_weights_pack_validation(lib):
    other = ctypes.c_void_p(0x2000)
    assert lib.moe_expert_weights_pack(0, 64, 64, FAKE, other, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_weights_pack(2, 64, 64, None, other, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_weights_pack(2, 64, 64, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG       # in place
    assert lib.moe_expert_weights_pack(2, 64, 64, ctypes.c_void_p(0x1008), other, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_weights_pack(2, 48, 64, FAKE, other, None) == L.MOE_ERR_UNSUPPORTED       # rows % 32
    assert lib.moe_expert_weights_pack(2, 64, 96, FAKE, other, None) == L.MOE_ERR_UNSUPPORTED       # cols % 64


def test_switch_layer_packed_weights_validation(lib):
    out = L.LayerOutputs()
    out.out = FAKE
    sh = _sh(m=64, d=64, n=8, xd=1)
    p = L.LayerParams(16, 0, 0, 0.01, None)
    p.weights_packed = 1                                           # identity expert: no weights to pack
    assert lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, None, None, None,
                                ctypes.byref(out), FAKE, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    p = L.LayerParams(16, 1, 64, 0.01, None)
    p.weights_packed = 1                                           # d = d_ff = 64: not on the stream kernel
    assert lib.moe_switch_layer(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None,
                                ctypes.byref(out), FAKE, 1 << 40, None) == L.MOE_ERR_UNSUPPORTED
    sv = L.LayerSaved(*([FAKE.value] * len(L.LayerSaved._fields_)))
    gr = L.LayerGrads(*([FAKE.value] * len(L.LayerGrads._fields_)))
    sh = _sh(m=64, d=256, n=8, xd=1)
    p = L.LayerParams(16, 1, 256, 0.01, None)
    p.weights_packed = 1                                           # the backward reads the plain layout
    assert lib.moe_switch_layer_backward(ctypes.byref(sh), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.byref(sv),
                                         FAKE, ctypes.byref(gr), FAKE, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
