"""Oracle: balanced optimal assignment (the LP of "MoE环游记：6") and its duals.

Test infrastructure only (see ``oracle/__init__.py``).

Follows [MoE tour 6]:
* "선형계획" eq. (3)/(4): maximise Σ_ij x_ij s_ij subject to Σ_j x_ij = k and
  Σ_i x_ij = mk/n (= q), with x in {0,1} (eq. 3) or [0,1] (eq. 4).
* "극대-극소" eq. (5)-(7): the Lagrangian swap; x*_ij = 1 where
  s_ij − α_i − β_j > 0, so the relaxation has the integer optimum.
* "분할정복" eq. (8)-(11): the reduced dual
  g(α, β) = Σ_ij max(0, s_ij − α_i − β_j) + k Σ α_i + q Σ β_j; for fixed β the
  best α_i is any value between the k-th and (k+1)-th largest of s_i − β,
  conventionally the (k+1)-th.
* "교대 반복" (Quantile Balancing): β = 0; repeat T times
  α_i ← (k+1)-th largest of s_i − β, β_j ← (q+1)-th largest of s_·j − α;
  output x_i = top-k of s_i − β.  The page's text of the β step names
  s_ij − β_j, its algorithm box s − α; the box is followed.
* "함정에 주의": the online form routes with the old β first, then makes one
  α update and one β update.

Precision: the Quantile-Balancing duals are exact order statistics of fp32
differences (fl32(s − β), fl32(s − α)), so ``qb_*`` work in fp32 and are
bit-reproducible.  ``qb_*`` take the exact order statistic of the algorithm
box.  With ``bip`` they take the BIP variant of "관련 연구" (eqs. (12)-(14)):
the inequality-constrained problem gives the same steps with each dual
truncated at zero, α ← max(0, ·) and β ← max(0, ·).

The quantile form (``quantile_*``) reads the last paragraph of "교대 반복":
the (k+1)-th largest of n and the (mk/n+1)-th largest of m are both the
1 − k/n quantile of their axis, and a framework quantile function may replace
the sort.  The demo ("데모 코드") uses numpy's default quantile, which places
the level at fractional position (N − 1)·level of the ascending values and
interpolates linearly between the two neighbours; on fp32 data numpy does
that arithmetic in fp32.  ``_interp_quantile_fp32`` states that rule.

Mini-batch β ("함정에 주의", last paragraph): when one column selection over
all m tokens is too expensive, the tokens are split into mini-batches, β is
computed on each by the same formula and the results are averaged.
``minibatch_beta`` takes contiguous row blocks and averages in fp64 in block
order, rounding once to fp32 (a reading: the page fixes neither the split
nor the precision of the mean).

Exact balance (reading): the alternating iteration stalls short of exact
column counts on skewed scores, while the pages' target is exactly q per
expert.  ``ssp_complete`` therefore finishes from the QB result with
successive shortest paths (min-cost flow) on the expert graph, in float64,
until every expert holds q tokens; the result is the LP optimum.  It is
checked against ``lp_highs`` (scipy's HiGHS on eq. (4)), against brute force
(``brute_force_*``) and against the dual objective eq. (8).
"""
from __future__ import annotations

import heapq
import itertools
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


# ------------------------------------------------------------------ QB (fp32, exact order statistics)
def _kth_largest_rows(v: np.ndarray, k: int) -> np.ndarray:
    """0-based k: the (k+1)-th largest of each row (des_sort(v, axis=1)[:, k])."""
    return -np.sort(-v, axis=1)[:, k]


def _truncate(v: np.ndarray, bip: bool) -> np.ndarray:
    """eq. (14): the BIP duals are kept non-negative, max(0, ·)."""
    return np.maximum(v, np.float32(0)).astype(np.float32) if bip else v


def qb_alpha(s: np.ndarray, beta: np.ndarray, k: int, bip: bool = False) -> np.ndarray:
    v = (s.astype(np.float32) - beta.astype(np.float32)[None, :]).astype(np.float32)
    return _truncate(_kth_largest_rows(v, k).astype(np.float32), bip)


def qb_beta(s: np.ndarray, alpha: np.ndarray, q: int, bip: bool = False) -> np.ndarray:
    w = (s.astype(np.float32) - alpha.astype(np.float32)[:, None]).astype(np.float32)
    return _truncate((-np.sort(-w, axis=0)[q, :]).astype(np.float32), bip)


def topk_biased(s: np.ndarray, beta: np.ndarray, k: int) -> np.ndarray:
    """x_i = top-k of fl32(s_i − β), lower expert index first on ties, by descending key."""
    v = (s.astype(np.float32) - beta.astype(np.float32)[None, :]).astype(np.float32)
    return np.argsort(-v, axis=1, kind="stable")[:, :k].astype(np.int32)


def qb_solve(s: np.ndarray, k: int, iters: int, beta0: Optional[np.ndarray] = None, bip: bool = False):
    """Quantile Balancing, solve form (BIP's truncated steps with ``bip``).
    Returns (idx [m,k], beta [n], alpha [m])."""
    m, n = s.shape
    q = m * k // n
    beta = np.zeros(n, np.float32) if beta0 is None else np.asarray(beta0, np.float32).copy()
    alpha = np.zeros(m, np.float32)
    for _ in range(iters):
        alpha = qb_alpha(s, beta, k, bip)
        beta = qb_beta(s, alpha, q, bip)
    return topk_biased(s, beta, k), beta, alpha


def qb_online(s: np.ndarray, k: int, beta_old: np.ndarray, bip: bool = False):
    """Online form: route with the old β, then one α and one β update."""
    m, n = s.shape
    q = m * k // n
    idx = topk_biased(s, beta_old, k)
    alpha = qb_alpha(s, beta_old, k, bip)
    beta = qb_beta(s, alpha, q, bip)
    return idx, beta, alpha


def bip_reduced_assignment(s: np.ndarray, alpha: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """eq. (7) at BIP duals: x_ij = 1 exactly where s_ij − α_i − β_j > 0 (float64).
    With α_i = 0 a row may hold fewer than k experts: the inequality form of eq. (12)
    lets a token leave a slot empty."""
    r = s.astype(np.float64) - np.asarray(alpha, np.float64)[:, None] - np.asarray(beta, np.float64)[None, :]
    return r > 0


def minibatch_beta(s: np.ndarray, k: int, iters: int, batch_rows: int, beta0: Optional[np.ndarray] = None,
                   bip: bool = False, quantile: bool = False) -> np.ndarray:
    """"함정에 주의", last paragraph: β computed on each mini-batch of ``batch_rows``
    consecutive tokens (its own q_b = batch_rows·k/n, ``iters`` QB steps from
    beta0, exact or quantile form), then averaged over the mini-batches.  Needs
    m % batch_rows == 0 and batch_rows·k % n == 0.  The mean is an fp64 sum in block
    order, divided by the number of blocks, rounded once to fp32."""
    m, n = s.shape
    if m % batch_rows or (batch_rows * k) % n:
        raise ValueError("mini-batches must tile the tokens and hold whole quotas")
    acc = np.zeros(n, np.float64)
    nb = m // batch_rows
    for b in range(nb):
        sb = s[b * batch_rows:(b + 1) * batch_rows]
        if quantile:
            _, beta_b, _ = qb_quantile_solve(sb, k, iters, bip, beta0)
        else:
            _, beta_b, _ = qb_solve(sb, k, iters, beta0, bip)
        acc = acc + beta_b.astype(np.float64)
    return (acc / nb).astype(np.float32)


# ------------------------------------------------------------------ QB, quantile form
def _interp_quantile_fp32(ascending: np.ndarray, level: np.float32) -> np.ndarray:
    """Linear-interpolation quantile along axis 0 of values sorted ascending, in fp32:
    position p = (N − 1)·level; below it the value at floor(p), above it the next one,
    weight g = p − floor(p).  The blend is a + (b − a)·g, or b − (b − a)·(1 − g) once
    g ≥ 1/2 (the form that stays exact at g = 1); at p ≥ N − 1 it is the maximum."""
    N = ascending.shape[0]
    pos = np.float32(N - 1) * np.float32(level)
    lo = int(np.floor(pos))
    if lo >= N - 1:
        return ascending[N - 1].astype(np.float32)
    g = np.float32(pos - np.float32(lo))
    a = ascending[lo].astype(np.float32)
    b = ascending[lo + 1].astype(np.float32)
    diff = (b - a).astype(np.float32)
    if g >= np.float32(0.5):
        return (b - (diff * np.float32(np.float32(1) - g)).astype(np.float32)).astype(np.float32)
    return (a + (diff * g).astype(np.float32)).astype(np.float32)


def _level(k: int, n: int) -> np.float32:
    """The common level 1 − k/n of both axes ("교대 반복"), as an fp32 number."""
    return np.float32(1.0 - k / n)


def quantile_alpha(s: np.ndarray, beta: np.ndarray, k: int, bip: bool = False) -> np.ndarray:
    """α_i = the 1 − k/n quantile of the row fl32(s_i − β) (rows sorted ascending)."""
    n = s.shape[1]
    v = (s.astype(np.float32) - beta.astype(np.float32)[None, :]).astype(np.float32)
    a = _interp_quantile_fp32(np.sort(v, axis=1).T, _level(k, n))
    return _truncate(a, bip)


def quantile_beta(s: np.ndarray, alpha: np.ndarray, k: int, bip: bool = False) -> np.ndarray:
    """β_j = the 1 − k/n quantile of the column fl32(s_·j − α)."""
    n = s.shape[1]
    w = (s.astype(np.float32) - alpha.astype(np.float32)[:, None]).astype(np.float32)
    b = _interp_quantile_fp32(np.sort(w, axis=0), _level(k, n))
    return _truncate(b, bip)


def qb_quantile_solve(s: np.ndarray, k: int, iters: int, bip: bool = False, beta0: Optional[np.ndarray] = None):
    """Alternating quantiles, iters rounds from β = 0 (or beta0); then the biased top-k.
    Returns (idx, beta, alpha)."""
    m, n = s.shape
    beta = np.zeros(n, np.float32) if beta0 is None else np.asarray(beta0, np.float32).copy()
    alpha = np.zeros(m, np.float32)
    for _ in range(iters):
        alpha = quantile_alpha(s, beta, k, bip)
        beta = quantile_beta(s, alpha, k, bip)
    return topk_biased(s, beta, k), beta, alpha


# ------------------------------------------------------------------ SignSGD on β
def dual_of_beta(s: np.ndarray, beta: np.ndarray, k: int) -> float:
    """ℓ(β) = Σ_i (sum of the k largest of s_i − β) + q Σ_j β_j in float64: eq. (8)
    with α at its best value for β ("분할정복"), which the gradient steps descend."""
    m, n = s.shape
    q = m * k // n
    v = s.astype(np.float64) - np.asarray(beta, np.float64)[None, :]
    top = -np.sort(-v, axis=1)[:, :k]
    return float(top.sum() + q * np.asarray(beta, np.float64).sum())


def signsgd_solve(s: np.ndarray, k: int, iters: int, gamma: float, beta0: Optional[np.ndarray] = None):
    """[MoE tour 6] "경사하강" eq. (15)-(17): β_j ← β_j − γ·sign(∂ℓ/∂β_j) with
    ∂ℓ/∂β_j = q − c_j, c_j the number of tokens whose top-k of fl32(s_i − β)
    holds j (reading: the page counts s_ij − α_i − β_j > 0 with α_i the
    (k+1)-th largest, the same set whenever a row's k-th and (k+1)-th values
    differ; ties go to the lower expert as in the routing).  fp32 update
    fl32(β_j + γ·sign(c_j − q)).  Returns (idx of the final β, beta, counts)."""
    m, n = s.shape
    q = m * k // n
    beta = np.zeros(n, np.float32) if beta0 is None else np.asarray(beta0, np.float32).copy()
    g = np.float32(gamma)
    for _ in range(iters):
        c = np.bincount(topk_biased(s, beta, k).ravel(), minlength=n)
        beta = (beta + g * np.sign(c - q).astype(np.float32)).astype(np.float32)
    idx = topk_biased(s, beta, k)
    return idx, beta, np.bincount(idx.ravel(), minlength=n).astype(np.int32)


# ------------------------------------------------------------------ assignments
def idx_to_x(idx: np.ndarray, n: int) -> np.ndarray:
    m = idx.shape[0]
    x = np.zeros((m, n), dtype=bool)
    x[np.arange(m)[:, None], idx] = True
    return x


def x_to_idx(x: np.ndarray, key: Optional[np.ndarray] = None) -> np.ndarray:
    """Selected experts per row; ordered by descending key (lower index on ties) if given."""
    m, n = x.shape
    k = int(x[0].sum())
    if key is None:
        key = np.zeros((m, n))
    k2 = np.where(x, key, -np.inf)
    return np.argsort(-k2, axis=1, kind="stable")[:, :k].astype(np.int32)


def objective(s: np.ndarray, x: np.ndarray) -> float:
    return float(np.sum(np.where(x, s.astype(np.float64), 0.0)))


def dual_objective(s: np.ndarray, alpha: np.ndarray, beta: np.ndarray, k: int) -> float:
    """eq. (8): Σ max(0, s − α − β) + k Σ α + q Σ β, float64."""
    m, n = s.shape
    q = m * k // n
    s64 = s.astype(np.float64)
    a = np.asarray(alpha, np.float64)
    b = np.asarray(beta, np.float64)
    r = np.maximum(0.0, s64 - a[:, None] - b[None, :])
    return float(r.sum() + k * a.sum() + q * b.sum())


def best_alpha(s: np.ndarray, beta: np.ndarray, k: int) -> np.ndarray:
    """eq. (11) in float64: α_i = (k+1)-th largest of s_i − β."""
    v = s.astype(np.float64) - np.asarray(beta, np.float64)[None, :]
    return _kth_largest_rows(v, k)


# ------------------------------------------------------------------ exact completion (SSP)
@dataclass
class Completion:
    x: np.ndarray          # [m, n] bool, column sums exactly q
    beta: np.ndarray       # [n] float64 potentials (an optimal dual)
    augmentations: int


def _move_costs(s64: np.ndarray, x: np.ndarray):
    """M[a, j] = min over tokens i with x_ia = 1, x_ij = 0 of s_ia − s_ij, and the token."""
    m, n = x.shape
    M = np.full((n, n), np.inf)
    arg = np.full((n, n), -1, dtype=np.int64)
    for a in range(n):
        toks = np.nonzero(x[:, a])[0]
        if toks.size == 0:
            continue
        cost = s64[toks, a][:, None] - s64[toks, :]
        cost[x[toks]] = np.inf
        best = np.argmin(cost, axis=0)          # first (lowest token index) on ties
        M[a] = cost[best, np.arange(n)]
        arg[a] = np.where(np.isfinite(M[a]), toks[best], -1)
    return M, arg


def ssp_complete(s: np.ndarray, k: int, beta: np.ndarray) -> Completion:
    """Exact LP optimum by successive shortest paths from x = top-k(s − β).

    Expert graph: an edge a → j moves one token from expert a to expert j at
    cost s_ia − s_ij (the cheapest such token).  Potentials start at β, for
    which x = top-k(s − β) gives non-negative reduced costs
    M(a,j) − π_a + π_j.  Each round runs Dijkstra from every over-full expert,
    stops at the first under-full expert reached, moves the tokens along that
    path and lowers the potentials by min(d, d_target).
    """
    m, n = s.shape
    q = m * k // n
    s64 = s.astype(np.float64)
    pi = np.asarray(beta, np.float64).copy()
    key = s64 - pi[None, :]
    x = idx_to_x(np.argsort(-key, axis=1, kind="stable")[:, :k], n)
    c = x.sum(axis=0).astype(np.int64)
    aug = 0
    while np.any(c > q):
        M, arg = _move_costs(s64, x)
        W = np.maximum(M - pi[:, None] + pi[None, :], 0.0)     # reduced costs (clip rounding)
        dist = np.full(n, np.inf)
        pred = np.full(n, -1, dtype=np.int64)
        done = np.zeros(n, dtype=bool)
        dist[c > q] = 0.0
        target = -1
        while True:
            cand = np.where(done, np.inf, dist)
            u = int(np.argmin(cand))
            if not np.isfinite(cand[u]):
                raise RuntimeError("no augmenting path")
            done[u] = True
            if c[u] < q:
                target = u
                break
            nd = dist[u] + W[u]
            better = (~done) & (nd < dist)
            dist[better] = nd[better]
            pred[better] = u
        D = dist[target]
        pi -= np.where(done, np.minimum(dist, D), D)
        # move one token along each edge of the path
        j = target
        while pred[j] >= 0:
            a = int(pred[j])
            i = int(arg[a, j])
            x[i, a] = False
            x[i, j] = True
            j = a
        c[j] -= 1
        c[target] += 1
        aug += 1
    return Completion(x, pi, aug)


# ------------------------------------------------------------------ LP via HiGHS
def lp_highs(s: np.ndarray, k: int):
    """eq. (4) solved by scipy's HiGHS.  Returns the (fractional) x and the objective."""
    from scipy.optimize import linprog
    from scipy.sparse import coo_matrix, vstack

    m, n = s.shape
    q = m * k // n
    rows = np.repeat(np.arange(m), n)
    cols = np.arange(m * n)
    A_row = coo_matrix((np.ones(m * n), (rows, cols)), shape=(m, m * n))
    rows2 = np.tile(np.arange(n), m)
    A_col = coo_matrix((np.ones(m * n), (rows2, cols)), shape=(n, m * n))
    A = vstack([A_row, A_col]).tocsr()
    b = np.concatenate([np.full(m, k, np.float64), np.full(n, q, np.float64)])
    res = linprog(-s.astype(np.float64).reshape(-1), A_eq=A, b_eq=b, bounds=(0.0, 1.0),
                  method="highs")
    if res.status != 0:
        raise RuntimeError(res.message)
    return res.x.reshape(m, n), -res.fun


def lp_highs_leq(s: np.ndarray, k: int):
    """The relaxation of BIP's problem eq. (12) ("관련 연구": Σ_j x_ij ≤ k and Σ_i x_ij ≤ mk/n,
    0 ≤ x ≤ 1) solved by scipy's HiGHS.  Returns (x, objective)."""
    from scipy.optimize import linprog
    from scipy.sparse import coo_matrix, vstack

    m, n = s.shape
    q = m * k // n
    cols = np.arange(m * n)
    A_row = coo_matrix((np.ones(m * n), (np.repeat(np.arange(m), n), cols)), shape=(m, m * n))
    A_col = coo_matrix((np.ones(m * n), (np.tile(np.arange(n), m), cols)), shape=(n, m * n))
    A = vstack([A_row, A_col]).tocsr()
    b = np.concatenate([np.full(m, k, np.float64), np.full(n, q, np.float64)])
    res = linprog(-s.astype(np.float64).reshape(-1), A_ub=A, b_ub=b, bounds=(0.0, 1.0), method="highs")
    if res.status != 0:
        raise RuntimeError(res.message)
    return res.x.reshape(m, n), -res.fun


# ------------------------------------------------------------------ brute force (tiny m, n)
def _choices(n: int, k: int):
    return [np.array(c, dtype=np.int64) for c in itertools.combinations(range(n), k)]


def brute_force_dp(s: np.ndarray, k: int) -> Tuple[int, float]:
    """Count of feasible {0,1} assignments and their best objective, by a DP over
    per-expert count vectors (exhaustive; tiny m, n only)."""
    m, n = s.shape
    q = m * k // n
    s64 = s.astype(np.float64)
    ch = _choices(n, k)
    states = {tuple([0] * n): (1, 0.0)}
    for i in range(m):
        nxt = {}
        for st, (cnt, best) in states.items():
            for c in ch:
                ns = list(st)
                ok = True
                for j in c:
                    ns[j] += 1
                    if ns[j] > q:
                        ok = False
                if not ok:
                    continue
                ns = tuple(ns)
                val = best + float(s64[i, c].sum())
                if ns in nxt:
                    c0, b0 = nxt[ns]
                    nxt[ns] = (c0 + cnt, max(b0, val))
                else:
                    nxt[ns] = (cnt, val)
        states = nxt
    cnt, best = states[tuple([q] * n)]
    return cnt, best


def brute_force_mitm(s: np.ndarray, k: int) -> Tuple[int, float, np.ndarray]:
    """Same count and optimum by meet-in-the-middle enumeration over the two halves of
    the tokens; also returns one optimal x."""
    m, n = s.shape
    q = m * k // n
    s64 = s.astype(np.float64)
    ch = _choices(n, k)
    h = m // 2

    def enum(lo, hi):
        table = {}
        for combo in itertools.product(range(len(ch)), repeat=hi - lo):
            cnt = np.zeros(n, dtype=np.int64)
            val = 0.0
            for t, ci in enumerate(combo):
                cnt[ch[ci]] += 1
                val += float(s64[lo + t, ch[ci]].sum())
            key = tuple(cnt)
            if key in table:
                c0, b0, a0 = table[key]
                table[key] = (c0 + 1, val, combo) if val > b0 else (c0 + 1, b0, a0)
            else:
                table[key] = (1, val, combo)
        return table

    A = enum(0, h)
    B = enum(h, m)
    total = 0
    best = -np.inf
    arg = None
    for key, (ca, ba, aa) in A.items():
        comp = tuple(q - v for v in key)
        if comp in B:
            cb, bb, ab = B[comp]
            total += ca * cb
            if ba + bb > best:
                best, arg = ba + bb, aa + ab
    x = np.zeros((m, n), dtype=bool)
    for i, ci in enumerate(arg):
        x[i, ch[ci]] = True
    return total, best, x
