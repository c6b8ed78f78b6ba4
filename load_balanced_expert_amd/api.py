"""Thin Python binding over libmoe's C ABI (include/moe.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the path runs in libmoe's HIP kernels.  Names follow
the C entry points (moe_route -> route, ...).  Outputs are allocated here
with torch.empty on the input's device; errors raise MoeError.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


class MoeError(RuntimeError):
    pass


def _lib():
    return L.load()


def _check(status: int, what: str):
    if status != L.MOE_OK:
        msg = _lib().moe_status_str(status).decode()
        raise MoeError(f"{what}: {msg} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise MoeError("libmoe takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _on_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MoeError("libmoe takes device tensors only")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.MOE_BF16
    if t.dtype == torch.float32:
        return L.MOE_F32
    raise MoeError(f"hidden states must be bf16 or fp32, got {t.dtype}")


def shape(m, d, n, k, score="softmax", gate="prob", x_dtype=L.MOE_BF16) -> L.MoeShape:
    return L.MoeShape(int(m), int(d), int(n), int(k), L.SCORES[score], L.GATES[gate], int(x_dtype))


# ------------------------------------------------------------------ workspace
_ws = {}


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-initialised uint8 device buffer of at least nbytes, cached per (device, current
    stream): calls on one stream run in order and may share it (the library leaves its control
    words zero), calls on different streams may overlap and get buffers of their own."""
    dev = torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            torch.cuda.current_stream(index).synchronize()   # the old buffer may still be in use
        buf = torch.zeros(max(int(nbytes), 1 << 16) + 256, dtype=torch.uint8, device=torch.device("cuda", index))
        _ws[key] = buf
    return buf


def _ws_args(nbytes: int, device):
    buf = workspace(nbytes, device)
    base = buf.data_ptr()
    aligned = (base + 255) // 256 * 256
    return ctypes.c_void_p(aligned), ctypes.c_size_t(buf.numel() - (aligned - base))


def capacity(m: int, n: int, cf: float) -> int:
    return int(_lib().moe_capacity(int(m), int(n), float(cf)))


def workspace_size(sh: L.MoeShape, capacity: int = -1, d_ff: int = 0) -> int:
    return int(_lib().moe_workspace_size(ctypes.byref(sh), int(capacity), int(d_ff)))


# ------------------------------------------------------------------ router
@dataclass
class RouteOut:
    idx: torch.Tensor
    gate: torch.Tensor
    counts: torch.Tensor
    prob_sum: Optional[torch.Tensor]


def router_prepare(w_r: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact three-way bf16 split of the fp32 router weight, reusable by route(w_planes=...)."""
    _on_device(w_r, out)
    d, n = w_r.shape
    nbytes = int(_lib().moe_router_planes_bytes(int(d), int(n)))
    planes = out if out is not None else torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w_r.device)
    if planes.numel() * planes.element_size() < nbytes:
        raise MoeError("router planes buffer too small")
    _check(_lib().moe_router_prepare(int(d), int(n), _ptr(w_r), _ptr(planes), _stream(w_r.device)),
           "moe_router_prepare")
    return planes


def route(x: torch.Tensor, w_r: torch.Tensor, k: int, score: str = "softmax", gate: str = "prob",
          bias: Optional[torch.Tensor] = None, prob_sum: bool = True, out: Optional[RouteOut] = None,
          w_planes: Optional[torch.Tensor] = None) -> RouteOut:
    _on_device(x, w_r, bias, w_planes)
    m, d = x.shape
    n = w_r.shape[1]
    dev = x.device
    sh = shape(m, d, n, k, score, gate, _dtype_code(x))
    if out is not None:
        idx, g, counts, ps = out.idx, out.gate, out.counts, out.prob_sum
    else:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
        g = torch.empty((m, k), dtype=torch.float32, device=dev)
        counts = torch.empty(n, dtype=torch.int32, device=dev)
        ps = torch.empty(n, dtype=torch.float32, device=dev) if prob_sum else None
    ws, wsb = _ws_args(workspace_size(sh), dev)
    _check(_lib().moe_route(ctypes.byref(sh), _ptr(x), _ptr(w_r), _ptr(w_planes), _ptr(bias), _ptr(idx), _ptr(g),
                            _ptr(counts), _ptr(ps), ws, wsb, _stream(dev)), "moe_route")
    return RouteOut(idx, g, counts, ps)


def route_lossfree(x: torch.Tensor, w_r: torch.Tensor, k: int, bias: torch.Tensor, gamma: float,
                   score: str = "sigmoid", gate: str = "prob", prob_sum: bool = True,
                   global_counts: Optional[torch.Tensor] = None, global_tokens: Optional[torch.Tensor] = None,
                   out: Optional[RouteOut] = None, w_planes: Optional[torch.Tensor] = None) -> RouteOut:
    """One Loss-Free micro-batch step through moe_route_lossfree: route with `bias`, then update `bias`
    in place (and add into global_counts / global_tokens when given) in the same launch; the results
    equal route() followed by stats(..., bias=bias, gamma=gamma)."""
    _on_device(x, w_r, bias, w_planes, global_counts, global_tokens)
    if bias is None:
        raise MoeError("route_lossfree needs the bias it updates")
    m, d = x.shape
    n = w_r.shape[1]
    dev = x.device
    sh = shape(m, d, n, k, score, gate, _dtype_code(x))
    if out is not None:
        idx, g, counts, ps = out.idx, out.gate, out.counts, out.prob_sum
    else:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
        g = torch.empty((m, k), dtype=torch.float32, device=dev)
        counts = torch.empty(n, dtype=torch.int32, device=dev)
        ps = torch.empty(n, dtype=torch.float32, device=dev) if prob_sum else None
    ws, wsb = _ws_args(workspace_size(sh), dev)
    _check(_lib().moe_route_lossfree(ctypes.byref(sh), _ptr(x), _ptr(w_r), _ptr(w_planes), _ptr(bias),
                                     float(gamma), _ptr(idx), _ptr(g), _ptr(counts), _ptr(ps),
                                     _ptr(global_counts), _ptr(global_tokens), ws, wsb, _stream(dev)),
           "moe_route_lossfree")
    return RouteOut(idx, g, counts, ps)


def route_noalloc(x: torch.Tensor, w_r: torch.Tensor, k: int, score: str = "softmax", gate: str = "prob",
                  bias: Optional[torch.Tensor] = None, prob_sum: bool = True, out: Optional[RouteOut] = None,
                  w_planes: Optional[torch.Tensor] = None) -> RouteOut:
    """route() through moe_route_noalloc: the library's static scratch instead of a workspace
    (outputs are allocated here unless `out` is given)."""
    _on_device(x, w_r, bias, w_planes)
    m, d = x.shape
    n = w_r.shape[1]
    dev = x.device
    sh = shape(m, d, n, k, score, gate, _dtype_code(x))
    if out is not None:
        idx, g, counts, ps = out.idx, out.gate, out.counts, out.prob_sum
    else:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
        g = torch.empty((m, k), dtype=torch.float32, device=dev)
        counts = torch.empty(n, dtype=torch.int32, device=dev)
        ps = torch.empty(n, dtype=torch.float32, device=dev) if prob_sum else None
    _check(_lib().moe_route_noalloc(ctypes.byref(sh), _ptr(x), _ptr(w_r), _ptr(w_planes), _ptr(bias), _ptr(idx),
                                    _ptr(g), _ptr(counts), _ptr(ps), _stream(dev)), "moe_route_noalloc")
    return RouteOut(idx, g, counts, ps)


# ------------------------------------------------------------------ statistics
@dataclass
class StatsOut:
    f: torch.Tensor
    P: Optional[torch.Tensor]
    aux: Optional[torch.Tensor]


def stats(m: int, k: int, counts: torch.Tensor, prob_sum: Optional[torch.Tensor], alpha: float = 1e-2,
          global_counts: Optional[torch.Tensor] = None, global_tokens: Optional[torch.Tensor] = None,
          bias: Optional[torch.Tensor] = None, gamma: float = 1e-3, out: Optional[StatsOut] = None) -> StatsOut:
    _on_device(counts, prob_sum, global_counts, global_tokens, bias)
    n = counts.shape[0]
    dev = counts.device
    if out is not None:
        f, P, aux = out.f, out.P, out.aux
    else:
        f = torch.empty(n, dtype=torch.float32, device=dev)
        P = torch.empty(n, dtype=torch.float32, device=dev) if prob_sum is not None else None
        aux = torch.empty(1, dtype=torch.float32, device=dev) if prob_sum is not None else None
    _check(_lib().moe_stats(int(m), int(n), int(k), _ptr(counts), _ptr(prob_sum), float(alpha), _ptr(f), _ptr(P),
                            _ptr(aux), _ptr(global_counts), _ptr(global_tokens), _ptr(bias), float(gamma),
                            _stream(dev)), "moe_stats")
    return StatsOut(f, P, aux)


def global_aux(global_counts: torch.Tensor, global_tokens: torch.Tensor, P_rows: torch.Tensor, alpha: float = 1e-2):
    n = global_counts.shape[0]
    nb = P_rows.shape[0]
    dev = global_counts.device
    fg = torch.empty(n, dtype=torch.float32, device=dev)
    losses = torch.empty(max(nb, 1), dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    _check(_lib().moe_global_aux(int(n), _ptr(global_counts), _ptr(global_tokens), _ptr(P_rows), int(nb),
                                 float(alpha), _ptr(fg), _ptr(losses), _ptr(mean), None, 0.0, 0.0, None, None,
                                 _stream(dev)), "moe_global_aux")
    return fg, losses[:nb], mean


def global_aux_hybrid(global_counts: torch.Tensor, global_tokens: torch.Tensor, P_rows: torch.Tensor,
                      micro_aux: torch.Tensor, alpha: float = 1e-2, global_weight: float = 1.0,
                      micro_weight: float = 1e-2):
    """(global losses [nb], hybrid losses [nb], hybrid mean [1]): global_weight times each
    micro-batch's global-batch loss plus micro_weight times its own Switch loss (micro_aux[t],
    as moe_stats returns it)."""
    _on_device(global_counts, global_tokens, P_rows, micro_aux)
    n = global_counts.shape[0]
    nb = P_rows.shape[0]
    dev = global_counts.device
    losses = torch.empty(max(nb, 1), dtype=torch.float32, device=dev)
    hybrid = torch.empty(max(nb, 1), dtype=torch.float32, device=dev)
    hmean = torch.empty(1, dtype=torch.float32, device=dev)
    _check(_lib().moe_global_aux(int(n), _ptr(global_counts), _ptr(global_tokens), _ptr(P_rows), int(nb),
                                 float(alpha), None, _ptr(losses), None, _ptr(micro_aux), float(global_weight),
                                 float(micro_weight),
                                 _ptr(hybrid), _ptr(hmean), _stream(dev)), "moe_global_aux")
    return losses[:nb], hybrid[:nb], hmean


# ------------------------------------------------------------------ balanced assignment
@dataclass
class BalanceOut:
    idx: torch.Tensor
    counts: torch.Tensor
    alpha: torch.Tensor
    info: torch.Tensor


def balance_duals(s: torch.Tensor, k: int, beta: torch.Tensor, iters: int = 5, mode: str = "solve",
                  exact: bool = False, quantile: bool = False, bip: bool = False) -> BalanceOut:
    """beta is updated in place.  quantile: the demo code's interpolated 1 - k/n quantiles;
    bip: α and β clipped at 0 after every step."""
    _on_device(s, beta)
    m, n = s.shape
    dev = s.device
    idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    alpha = torch.empty(m, dtype=torch.float32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    need = int(_lib().moe_balance_workspace_size(int(m), int(n), int(k), int(exact)))
    ws, wsb = _ws_args(need, dev)
    flags = (L.QB_QUANTILE if quantile else 0) | (L.QB_BIP if bip else 0)
    _check(_lib().moe_balance_duals(int(m), int(n), int(k), _ptr(s), _ptr(beta), int(iters), L.QB_MODES[mode] | flags,
                                    int(exact), _ptr(idx), _ptr(counts), _ptr(alpha), _ptr(info), ws, wsb,
                                    _stream(dev)), "moe_balance_duals")
    return BalanceOut(idx, counts, alpha, info)


def balance_duals_minibatch(s: torch.Tensor, k: int, beta: torch.Tensor, batch_rows: int, iters: int = 5,
                            mode: str = "solve", quantile: bool = False, bip: bool = False) -> BalanceOut:
    """β from mini-batches of batch_rows consecutive tokens, averaged (beta updated in place)."""
    _on_device(s, beta)
    m, n = s.shape
    dev = s.device
    idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    alpha = torch.empty(m, dtype=torch.float32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    need = int(_lib().moe_balance_minibatch_workspace_size(int(m), int(n), int(k), int(batch_rows)))
    ws, wsb = _ws_args(need, dev)
    flags = (L.QB_QUANTILE if quantile else 0) | (L.QB_BIP if bip else 0)
    _check(_lib().moe_balance_duals_minibatch(int(m), int(n), int(k), _ptr(s), _ptr(beta), int(iters),
                                              L.QB_MODES[mode] | flags, int(batch_rows), _ptr(idx), _ptr(counts),
                                              _ptr(alpha), _ptr(info), ws, wsb, _stream(dev)),
           "moe_balance_duals_minibatch")
    return BalanceOut(idx, counts, alpha, info)


def balance_signsgd(s: torch.Tensor, k: int, beta: torch.Tensor, gamma: float, iters: int):
    """Sign-gradient steps on β (updated in place); returns (idx, counts) of the final β."""
    _on_device(s, beta)
    m, n = s.shape
    dev = s.device
    idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    need = int(_lib().moe_balance_workspace_size(int(m), int(n), int(k), 0))
    ws, wsb = _ws_args(need, dev)
    _check(_lib().moe_balance_signsgd(int(m), int(n), int(k), _ptr(s), _ptr(beta), float(gamma), int(iters),
                                      _ptr(idx), _ptr(counts), ws, wsb, _stream(dev)), "moe_balance_signsgd")
    return idx, counts


# ------------------------------------------------------------------ dispatch
@dataclass
class DispatchOut:
    token_to_row: torch.Tensor
    drop_mask: torch.Tensor
    expert_offsets: torch.Tensor
    expert_rows: torch.Tensor
    row_to_token: torch.Tensor
    dispatched: Optional[torch.Tensor]


def dispatch_rows(m: int, k: int, n: int, capacity: int) -> int:
    """Rows of the dispatched buffer: capacity-padded n * C, or m * k without a capacity."""
    return m * k if capacity < 0 else capacity * n


def dispatch(x: Optional[torch.Tensor], idx: torch.Tensor, n: int, capacity: int = -1, d: Optional[int] = None,
             copy_rows: bool = True, out: Optional[DispatchOut] = None) -> DispatchOut:
    _on_device(x, idx)
    m, k = idx.shape
    dev = idx.device
    if x is not None:
        d = x.shape[1]
        xd = _dtype_code(x)
    else:
        xd = L.MOE_BF16
    sh = shape(m, d or 1, n, k, x_dtype=xd)
    rows_bound = dispatch_rows(m, k, n, capacity)
    if out is not None:
        t2r, drop, offs, rows, r2t, disp = (out.token_to_row, out.drop_mask, out.expert_offsets, out.expert_rows,
                                            out.row_to_token, out.dispatched)
    else:
        t2r = torch.empty((m, k), dtype=torch.int32, device=dev)
        drop = torch.empty((m, k), dtype=torch.uint8, device=dev)
        offs = torch.empty(n + 1, dtype=torch.int32, device=dev)
        rows = torch.empty(n, dtype=torch.int32, device=dev)
        r2t = torch.full((rows_bound,), -1, dtype=torch.int32, device=dev)
        disp = (torch.zeros((rows_bound, d), dtype=x.dtype, device=dev)
                if (x is not None and copy_rows) else None)
    ws, wsb = _ws_args(workspace_size(sh, capacity), dev)
    _check(_lib().moe_dispatch(ctypes.byref(sh), int(capacity), _ptr(x), _ptr(idx), _ptr(t2r), _ptr(drop),
                               _ptr(offs), _ptr(rows), _ptr(r2t), _ptr(disp), ws, wsb, _stream(dev)), "moe_dispatch")
    return DispatchOut(t2r, drop, offs, rows, r2t, disp)


# ------------------------------------------------------------------ expert FFN
def expert_ffn(dispatched: torch.Tensor, expert_offsets: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
               rows_max: int, out: Optional[torch.Tensor] = None,
               expert_rows: Optional[torch.Tensor] = None) -> torch.Tensor:
    """expert_rows: rows per expert (capacity-padded layout); None: compact offsets."""
    _on_device(dispatched, expert_offsets, w1, w2, expert_rows)
    n, d_ff, d = w1.shape
    dev = dispatched.device
    y = out if out is not None else torch.empty((dispatched.shape[0], d), dtype=torch.bfloat16, device=dev)
    need = int(_lib().moe_expert_ffn_workspace_size(int(n), int(rows_max), int(d_ff)))
    ws, wsb = _ws_args(need, dev)
    _check(_lib().moe_expert_ffn(int(n), int(d), int(d_ff), int(rows_max), _ptr(expert_offsets), _ptr(expert_rows),
                                 _ptr(dispatched), _ptr(w1), _ptr(w2), _ptr(y), ws, wsb, _stream(dev)),
           "moe_expert_ffn")
    return y


def pack_expert_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[n, rows, cols] bf16 expert weights (w1 or w2, Linear layout) rewritten in the order the FFN's
    weight-stream kernel reads them (moe_expert_weights_pack); same shape and values."""
    _on_device(w)
    if w.dtype != torch.bfloat16 or w.dim() != 3 or not w.is_contiguous():
        raise MoeError("pack_expert_weights takes a contiguous [n, rows, cols] bf16 tensor")
    n, rows, cols = w.shape
    p = out if out is not None else torch.empty_like(w)
    _check(_lib().moe_expert_weights_pack(int(n), int(rows), int(cols), _ptr(w), _ptr(p), _stream(w.device)),
           "moe_expert_weights_pack")
    return p


# ------------------------------------------------------------------ combine
def combine(y: torch.Tensor, gate: torch.Tensor, token_to_row: torch.Tensor, residual: Optional[torch.Tensor],
            out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _on_device(y, gate, token_to_row, residual)
    m, k = token_to_row.shape
    dev = y.device
    d = y.shape[1]
    odt = residual.dtype if residual is not None else (out_dtype or torch.float32)
    sh = shape(m, d, k, k, x_dtype=L.MOE_BF16 if odt == torch.bfloat16 else L.MOE_F32)
    if out is None:
        out = torch.empty((m, d), dtype=odt, device=dev)
    _check(_lib().moe_combine(ctypes.byref(sh), _ptr(y), _dtype_code(y), _ptr(gate), _ptr(token_to_row),
                              _ptr(residual), _ptr(out), _stream(dev)), "moe_combine")
    return out


# ------------------------------------------------------------------ whole layer
@dataclass
class LayerOut:
    idx: torch.Tensor
    gate: torch.Tensor
    counts: torch.Tensor
    prob_sum: torch.Tensor
    f: torch.Tensor
    P: torch.Tensor
    aux: torch.Tensor
    token_to_row: torch.Tensor
    drop_mask: torch.Tensor
    expert_offsets: torch.Tensor
    expert_rows: torch.Tensor
    row_to_token: torch.Tensor
    dispatched: torch.Tensor
    y: Optional[torch.Tensor]
    out: torch.Tensor
    hidden: Optional[torch.Tensor] = None   # [rows, d_ff] bf16 (relu_ffn), kept for the backward


def allocate_layer_outputs(m, d, n, k, rows_bound, x_dtype, ffn: bool, device, d_ff: Optional[int] = None) -> LayerOut:
    """Layer output buffers; with d_ff the relu_ffn hidden activation is kept too (for the backward)."""
    e = lambda *s, dt: torch.empty(s, dtype=dt, device=device)  # noqa: E731
    return LayerOut(
        idx=e(m, k, dt=torch.int32), gate=e(m, k, dt=torch.float32), counts=e(n, dt=torch.int32),
        prob_sum=e(n, dt=torch.float32), f=e(n, dt=torch.float32), P=e(n, dt=torch.float32),
        aux=e(1, dt=torch.float32), token_to_row=e(m, k, dt=torch.int32), drop_mask=e(m, k, dt=torch.uint8),
        expert_offsets=e(n + 1, dt=torch.int32), expert_rows=e(n, dt=torch.int32),
        row_to_token=torch.full((rows_bound,), -1, dtype=torch.int32, device=device),
        dispatched=e(rows_bound, d, dt=x_dtype), y=e(rows_bound, d, dt=torch.bfloat16) if ffn else None,
        out=e(m, d, dt=x_dtype), hidden=e(rows_bound, d_ff, dt=torch.bfloat16) if (ffn and d_ff) else None)


def switch_layer(x: torch.Tensor, w_r: torch.Tensor, k: int = 1, capacity: int = -1, alpha: float = 1e-2,
                 w1: Optional[torch.Tensor] = None, w2: Optional[torch.Tensor] = None,
                 bias: Optional[torch.Tensor] = None, score: str = "softmax", gate: str = "prob",
                 outputs: Optional[LayerOut] = None, stage_events=None, update_bias: bool = False,
                 gamma: float = 1e-3, global_counts: Optional[torch.Tensor] = None,
                 global_tokens: Optional[torch.Tensor] = None, weights_packed: bool = False) -> LayerOut:
    """stage_events: optional list of 6 torch.cuda.Event (timing enabled) recorded at the stage
    boundaries (start, router prepared, routed, dispatched, expert done, combined).
    update_bias: the layer routes with `bias`, then updates it in place (Loss-Free, rate gamma);
    global_counts / global_tokens (int64, both or neither) accumulate the global batch.
    weights_packed: w1 and w2 come from pack_expert_weights (same shapes, packed order)."""
    _on_device(x, w_r, w1, w2, bias, global_counts, global_tokens)
    if update_bias and bias is None:
        raise MoeError("update_bias needs the bias it updates")
    m, d = x.shape
    n = w_r.shape[1]
    dev = x.device
    ffn = w1 is not None
    d_ff = w1.shape[1] if ffn else 0
    sh = shape(m, d, n, k, score, gate, _dtype_code(x))
    rows_bound = dispatch_rows(m, k, n, capacity)
    o = outputs or allocate_layer_outputs(m, d, n, k, rows_bound, x.dtype, ffn, dev, d_ff if ffn else None)
    lo = L.LayerOutputs(*[(_ptr(getattr(o, f)) if getattr(o, f) is not None else None)
                          for f, _ in L.LayerOutputs._fields_])
    evs = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise MoeError("stage_events takes 6 events")
        if any(e is not None and not e.cuda_event for e in stage_events):
            raise MoeError("stage_events must be created first (record each event once)")
        evs = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e.cuda_event) if e is not None else None
                                      for e in stage_events])
    params = L.LayerParams(int(capacity), L.EXPERTS["relu_ffn" if ffn else "identity"], int(d_ff), float(alpha),
                           ctypes.cast(evs, ctypes.POINTER(ctypes.c_void_p)) if evs is not None else None,
                           _ptr(bias) if update_bias else None, float(gamma), _ptr(global_counts),
                           _ptr(global_tokens), int(bool(weights_packed)))
    ws, wsb = _ws_args(workspace_size(sh, capacity, d_ff), dev)
    _check(_lib().moe_switch_layer(ctypes.byref(sh), ctypes.byref(params), _ptr(x), _ptr(w_r), _ptr(w1), _ptr(w2),
                                   _ptr(bias), ctypes.byref(lo), ws, wsb, _stream(dev)), "moe_switch_layer")
    return o


# ------------------------------------------------------------------ backward
@dataclass
class LayerGrads:
    dx: torch.Tensor
    dw_r: torch.Tensor
    dw1: torch.Tensor
    dw2: torch.Tensor


def switch_layer_backward(x: torch.Tensor, w_r: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, fwd: LayerOut,
                          dout: torch.Tensor, capacity: int = -1, alpha: float = 1e-2,
                          out: Optional[LayerGrads] = None) -> LayerGrads:
    """Gradients of sum(out * dout) + aux for the forward `fwd` (its saved outputs, hidden included)."""
    _on_device(x, w_r, w1, w2, dout)
    if fwd.hidden is None or fwd.y is None:
        raise MoeError("the backward needs the forward's hidden activation and expert outputs")
    m, d = x.shape
    n = w_r.shape[1]
    k = fwd.idx.shape[1]
    d_ff = w1.shape[1]
    dev = x.device
    sh = shape(m, d, n, k, "softmax", "prob", _dtype_code(x))
    g = out or LayerGrads(torch.empty((m, d), dtype=torch.float32, device=dev),
                          torch.empty((d, n), dtype=torch.float32, device=dev),
                          torch.empty(tuple(w1.shape), dtype=torch.float32, device=dev),
                          torch.empty(tuple(w2.shape), dtype=torch.float32, device=dev))
    saved = L.LayerSaved(_ptr(fwd.idx), _ptr(fwd.gate), _ptr(fwd.counts), _ptr(fwd.token_to_row),
                         _ptr(fwd.expert_offsets), _ptr(fwd.expert_rows) if capacity >= 0 else None,
                         _ptr(fwd.dispatched), _ptr(fwd.hidden), _ptr(fwd.y))
    grads = L.LayerGrads(_ptr(g.dx), _ptr(g.dw_r), _ptr(g.dw1), _ptr(g.dw2))
    params = L.LayerParams(int(capacity), L.EXPERTS["relu_ffn"], int(d_ff), float(alpha), None)
    need = int(_lib().moe_switch_layer_backward_workspace_size(ctypes.byref(sh), int(capacity), int(d_ff)))
    ws, wsb = _ws_args(need, dev)
    _check(_lib().moe_switch_layer_backward(ctypes.byref(sh), ctypes.byref(params), _ptr(x), _ptr(w_r), _ptr(w1),
                                            _ptr(w2), ctypes.byref(saved), _ptr(dout), ctypes.byref(grads), ws, wsb,
                                            _stream(dev)), "moe_switch_layer_backward")
    return g
