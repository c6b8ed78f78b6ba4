"""Oracle: backward pass of the Switch layer (router, load-balancing loss, capacity dispatch,
ReLU expert FFN, gate-scaled combine with the residual), float64.

Test infrastructure only (see ``oracle/__init__.py``).

Follows
* [Switch review] "Switch Routing 메커니즘" Step 3: the expert output is multiplied by the
  router probability of the chosen expert, which is what lets the gradient reach W_r.
* [Switch impl] "argmax가 있어도 Router를 학습할 수 있는 이유": the chosen expert id is a
  discrete value that ordinary differentiation cannot move; the gradient flows through the
  continuous gate that multiplies the output.
* [Switch review] "로드 밸런싱 손실", "왜 f_i·P_i인가": f_i comes from the argmax and carries
  no gradient; P_i, the mean softmax probability, does.  L_aux = α·N·Σ_i f_i·P_i.
* [Switch review] "Switch Layer의 구조": FFN(x) = max(0, x·W1)·W2 per expert (no biases here).

Layer (as the forward oracle computes it): h = x·W_r, p = softmax(h), i*(t) = the token's chosen
expert(s) (given: the forward's selection), g(t, r) = p_{i_r}(t); kept pairs are dispatched to
capacity rows; A = D·W1ᵀ (w1 layout [d_ff, d]), H = max(0, A), Y = H·W2ᵀ (w2 layout [d, d_ff]);
out[t] = x[t] + Σ_r g(t, r)·Y[row(t, r)].  The scalar whose gradient is taken is
L = Σ out ⊙ dout + L_aux (dout: the gradient arriving from above).

Gradients, by the chain rule (reading: gate = the chosen expert's probability, softmax scores,
as in the Switch layer; the bf16 roundings of the forward's H and Y are kept when
``rounded=True``, so that the expert path is differentiated at the forward's saved values):
  dY[row]   = g·dout[t]                    (the combine's transpose)
  dg(t, r)  = <dout[t], Y[row]>
  dH        = dY·w2,  dA = dH ⊙ [A > 0],   dD = dA·w1
  dw2       = dYᵀ·H,  dw1 = dAᵀ·D          (in the weights' own layouts)
  dx_expert[t] = Σ_r dD[row(t, r)]         (the dispatch's transpose)
  c_j       = α·N·f_j / T                  (∂L_aux/∂p_j(t), the same for every token)
  dh(t)     = Σ_r dg(t, r)·g(t, r)·(e_{i_r} − p(t)) + p(t) ⊙ (c − <p(t), c>)   (softmax Jacobian)
  dW_r      = xᵀ·dh,  dx_router = dh·W_rᵀ
  dx        = dout + dx_expert + dx_router
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import expert as E
from . import router as R


@dataclass
class LayerGrads:
    dx: np.ndarray      # [T, d]
    dw_r: np.ndarray    # [d, N]
    dw1: np.ndarray     # [N, d_ff, d]  (zero for experts with no rows)
    dw2: np.ndarray     # [N, d, d_ff]
    dh: np.ndarray      # [T, N] gradient of the logits
    dgate: np.ndarray   # [T, k]  (0 for dropped pairs)


def _expert_forward(D: np.ndarray, w1: np.ndarray, w2: np.ndarray, rounded: bool):
    """A = D·W1ᵀ, H = max(0, A), Y = H·W2ᵀ for one expert (float64; bf16 roundings of H and Y as
    the forward stores them when rounded)."""
    W1 = E.from_bf16_bits(w1) if w1.dtype == np.uint16 else np.asarray(w1, np.float64)
    W2 = E.from_bf16_bits(w2) if w2.dtype == np.uint16 else np.asarray(w2, np.float64)
    A = D @ W1.T
    H = np.maximum(A, 0.0)
    if rounded:
        H = E.bf16_round(H)
    Y = H @ W2.T
    if rounded:
        Y = E.bf16_round(Y)
    return A, H, Y, W1, W2


def switch_layer_backward(x, w_r, idx, token_to_row, expert_offsets, expert_rows, w1, w2, dout, alpha: float,
                          counts=None, rounded: bool = True, wgrad_experts=None) -> LayerGrads:
    """Gradients of L = Σ out ⊙ dout + L_aux for one Switch layer forward, given its selection
    (idx [T, k]), its dispatch maps and the expert weights (bf16 bits or float arrays).
    wgrad_experts: the experts whose weight gradients are returned (dw1 / dw2 then hold those,
    in that order); None = all."""
    x64 = R.decode_hidden(x)
    T, d = x64.shape
    w_r64 = np.asarray(w_r, np.float64)
    N = w_r64.shape[1]
    idx = np.asarray(idx, np.int64)
    k = idx.shape[1]
    dout = np.asarray(dout, np.float64)
    h = x64 @ w_r64
    p = R.softmax(h)
    g = np.take_along_axis(p, idx, axis=1)                      # [T, k]
    if counts is None:
        counts = np.bincount(idx.ravel(), minlength=N)
    f = np.asarray(counts, np.float64) / T                      # f_j: no gradient
    c = alpha * N * f / T                                       # dL_aux / dp_j(t)

    dx = dout.copy()
    dgate = np.zeros((T, k))
    wl = list(range(N)) if wgrad_experts is None else [int(e) for e in wgrad_experts]
    slot = {e: i for i, e in enumerate(wl)}
    dw1 = np.zeros((len(wl),) + np.shape(w1)[1:])
    dw2 = np.zeros((len(wl),) + np.shape(w2)[1:])
    t2r = np.asarray(token_to_row)
    for e in range(N):
        lo, n_e = int(expert_offsets[e]), int(expert_rows[e])
        if n_e == 0:
            continue
        rows = np.arange(lo, lo + n_e)
        # the (token, choice) pair of every row of this expert
        pt, pr = np.nonzero(np.isin(t2r, rows))
        order = np.argsort(t2r[pt, pr])
        pt, pr = pt[order], pr[order]
        D = x64[pt]
        A, H, Y, W1, W2 = _expert_forward(D, w1[e], w2[e], rounded)
        dY = g[pt, pr][:, None] * dout[pt]
        dgate[pt, pr] = np.sum(dout[pt] * Y, axis=1)
        dH = dY @ W2
        dA = dH * (A > 0)
        dD = dA @ W1
        if e in slot:
            dw2[slot[e]] = dY.T @ H
            dw1[slot[e]] = dA.T @ D
        np.add.at(dx, pt, dD)
    # softmax Jacobian: gate term plus the balancing-loss term
    dh = p * (c[None, :] - np.sum(p * c[None, :], axis=1, keepdims=True))
    for r in range(k):
        coef = dgate[:, r] * g[:, r]
        dh -= coef[:, None] * p
        dh[np.arange(T), idx[:, r]] += coef
    dw_r = x64.T @ dh
    dx += dh @ w_r64.T
    return LayerGrads(dx, dw_r, dw1, dw2, dh, dgate)


def switch_layer_loss(x64, w_r64, idx, token_to_row, expert_offsets, expert_rows, w1, w2, dout, alpha: float,
                      counts) -> float:
    """The scalar L = Σ out ⊙ dout + α·N·Σ_j f_j·P_j in float64 with no bf16 roundings, written
    directly from the forward definitions (used to check the gradients by central differences;
    the selection and the dispatch maps are held fixed)."""
    T, d = x64.shape
    N = w_r64.shape[1]
    p = R.softmax(x64 @ w_r64)
    out = x64.copy()
    t2r = np.asarray(token_to_row)
    for e in range(N):
        lo, n_e = int(expert_offsets[e]), int(expert_rows[e])
        for row in range(lo, lo + n_e):
            t, r = [int(v[0]) for v in np.nonzero(t2r == row)]
            hid = np.maximum(x64[t] @ np.asarray(w1[e], np.float64).T, 0.0)
            y = hid @ np.asarray(w2[e], np.float64).T
            out[t] += p[t, idx[t, r]] * y
    f = np.asarray(counts, np.float64) / T
    P = p.mean(axis=0)
    return float(np.sum(out * dout) + alpha * N * np.sum(f * P))
