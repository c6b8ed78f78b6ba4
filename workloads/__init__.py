"""Seeded synthetic inputs for the MoE routing / balancing / dispatch path.

This module is the only code shared by the CPU oracle (``oracle/``) and the GPU
path (``load_balanced_expert_amd``).  It holds random draws and storage-format
conversion only (fp32 -> bf16 round-to-nearest-even of *generated inputs*);
none of the method's arithmetic lives here.

Every generator is a pure function of ``(spec, seed)``: numpy ``PCG64`` streams
derived from ``SeedSequence(seed, spawn_key=(stream, ...))`` so that any part
(for example one expert's FFN weights) can be regenerated on its own.

Workload shapes follow the setups the pages describe:

* Switch layers (top-1 softmax router, capacity factor, ReLU expert FFN):
  "Switch Transformers 논문 리뷰" (tildalice.io), sections "Switch Layer의 구조",
  "Switch Routing 메커니즘" and "Expert Capacity와 토큰 드롭"; the Switch-Base
  expert count (128) and the Switch-C expert count (2048) come from the same
  page's scaling section and from "Switch Transformer를 구현 관점에서 읽기"
  (molayo1419.me).
* Loss-Free biased top-k with per-domain skewed micro-batches: "MoE环游记：6"
  (kexue.fm/archives/11619), section "방법 회고" eq. (1)-(2), and the Qwen
  global-batch page (agentlenshq.com), section "마이크로-배치 로드 밸런스의 한계"
  (a micro-batch often holds one domain only).
* Balanced assignment scores with a per-expert offset (plain top-k is
  unbalanced): "MoE环游记：6", sections "선형계획" and "데모 코드" (the demo
  adds a per-expert uniform offset to uniform scores).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

# stream ids for SeedSequence spawn keys
_S_TOKENS, _S_ROUTER, _S_EXPERT, _S_MICRO, _S_SCORES, _S_IDX, _S_MISC = range(7)


def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


# ---------------------------------------------------------------- storage formats
def bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- specs
@dataclass(frozen=True)
class SwitchSpec:
    """One router + capacity + expert layer workload."""
    name: str
    T: int                      # tokens (batch x sequence flattened)
    d: int                      # d_model
    N: int                      # experts
    k: int = 1                  # experts per token
    score: str = "softmax"      # "softmax" | "sigmoid"
    x_dtype: str = "bf16"       # storage dtype of the hidden states
    x_std: float = 1.0
    w_r_std: float = 0.02
    capacity_factors: Tuple[float, ...] = (1.25,)
    d_ff: Optional[int] = None  # None: identity expert
    w_std: float = 0.0          # std of W1 and W2 entries (bf16)
    alpha: float = 1e-2         # aux-loss weight

    def capacity(self, cf: float) -> int:
        return int(math.floor(self.T * cf / self.N))

    def scaled(self, **kw) -> "SwitchSpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class LossFreeSpec:
    name: str = "lossfree_topk"
    micro_batches: int = 16
    T: int = 4096
    d: int = 2048
    N: int = 256
    k: int = 8
    clusters: int = 4
    mean_std: float = 2.0       # cluster means ~ N(0, 4) per dimension (variance 4)
    noise_std: float = 1.0
    w_r_std: float = 0.1 / math.sqrt(2048)
    gamma: float = 1e-3

    def scaled(self, **kw) -> "LossFreeSpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class BalancedSpec:
    name: str = "balanced_lp"
    m: int = 4096
    n: int = 64
    k: int = 4
    offset_std: float = 1.5
    noise_std: float = 1.0

    @property
    def q(self) -> int:
        return self.m * self.k // self.n

    def scaled(self, **kw) -> "BalancedSpec":
        return replace(self, **kw)


TINY_SWITCH = SwitchSpec("tiny_switch", T=1024, d=64, N=8, x_dtype="f32", w_r_std=0.02,
                         capacity_factors=(1.25,), d_ff=None)
SWITCH_BASE = SwitchSpec("switch_base", T=8192, d=768, N=128, x_dtype="bf16",
                         w_r_std=0.1 / math.sqrt(768), capacity_factors=(1.0, 1.25),
                         d_ff=3072, w_std=math.sqrt(1.0 / 768))
LOSSFREE = LossFreeSpec()
BALANCED = BalancedSpec()
SWITCH_C = SwitchSpec("switch_c", T=65536, d=1024, N=2048, x_dtype="bf16",
                      w_r_std=0.1 / math.sqrt(1024), capacity_factors=(1.25,),
                      d_ff=4096, w_std=math.sqrt(1.0 / 1024))


# ---------------------------------------------------------------- Switch layer inputs
@dataclass
class SwitchInputs:
    spec: SwitchSpec
    seed: int
    x: np.ndarray        # [T, d] float32, or uint16 bf16 bits
    w_r: np.ndarray      # [d, N] float32

    @property
    def x_is_bf16(self) -> bool:
        return self.x.dtype == np.uint16


def switch_inputs(spec: SwitchSpec, seed: int) -> SwitchInputs:
    """Hidden states x ~ N(0, x_std^2) then router weight W_r ~ N(0, w_r_std^2), fp32."""
    g = _gen(seed, _S_TOKENS)
    x = g.standard_normal((spec.T, spec.d), dtype=np.float32)
    if spec.x_std != 1.0:
        x *= np.float32(spec.x_std)
    if spec.x_dtype == "bf16":
        x = bf16_bits(x)
    gw = _gen(seed, _S_ROUTER)
    w_r = gw.standard_normal((spec.d, spec.N), dtype=np.float32) * np.float32(spec.w_r_std)
    return SwitchInputs(spec, seed, x, w_r.astype(np.float32))


def expert_weights(spec: SwitchSpec, seed: int, j: int):
    """Expert j's FFN weights as bf16 bits, in Linear (out x in) layout.

    w1: [d_ff, d]  (row f = weights feeding hidden unit f; math W1 = w1^T)
    w2: [d, d_ff]  (row c = weights feeding output channel c; math W2 = w2^T)
    """
    g = _gen(seed, _S_EXPERT, j)
    w1 = g.standard_normal((spec.d_ff, spec.d), dtype=np.float32) * np.float32(spec.w_std)
    w2 = g.standard_normal((spec.d, spec.d_ff), dtype=np.float32) * np.float32(spec.w_std)
    return bf16_bits(w1), bf16_bits(w2)


def all_expert_weights(spec: SwitchSpec, seed: int, threads: int = 8):
    """Stacked [N, d_ff, d] and [N, d, d_ff] bf16 bits (host memory; fine up to a few GB)."""
    from concurrent.futures import ThreadPoolExecutor
    w1 = np.empty((spec.N, spec.d_ff, spec.d), np.uint16)
    w2 = np.empty((spec.N, spec.d, spec.d_ff), np.uint16)

    def one(j):
        a, b = expert_weights(spec, seed, j)
        w1[j] = a
        w2[j] = b

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(spec.N)))
    return w1, w2


# ---------------------------------------------------------------- Loss-Free micro-batches
@dataclass
class LossFreeInputs:
    spec: LossFreeSpec
    seed: int
    means: np.ndarray    # [clusters, d] float32
    w_r: np.ndarray      # [d, N] float32

    def micro_batch(self, t: int) -> np.ndarray:
        """bf16 bits [T, d]: cluster (t mod clusters) mean + N(0, noise_std^2)."""
        s = self.spec
        g = _gen(self.seed, _S_MICRO, t)
        x = g.standard_normal((s.T, s.d), dtype=np.float32)
        if s.noise_std != 1.0:
            x *= np.float32(s.noise_std)
        x += self.means[t % s.clusters][None, :]
        return bf16_bits(x)


def lossfree_inputs(spec: LossFreeSpec, seed: int) -> LossFreeInputs:
    g = _gen(seed, _S_TOKENS)
    means = g.standard_normal((spec.clusters, spec.d), dtype=np.float32) * np.float32(spec.mean_std)
    gw = _gen(seed, _S_ROUTER)
    w_r = gw.standard_normal((spec.d, spec.N), dtype=np.float32) * np.float32(spec.w_r_std)
    return LossFreeInputs(spec, seed, means.astype(np.float32), w_r.astype(np.float32))


# ---------------------------------------------------------------- balanced-assignment scores
def balanced_scores(spec: BalancedSpec, seed: int) -> np.ndarray:
    """s_ij = o_j + eps_ij (summed in fp32), o ~ N(0, offset_std^2), eps ~ N(0, noise_std^2)."""
    g = _gen(seed, _S_SCORES)
    o = g.standard_normal(spec.n, dtype=np.float32) * np.float32(spec.offset_std)
    e = g.standard_normal((spec.m, spec.n), dtype=np.float32) * np.float32(spec.noise_std)
    return (e + o[None, :]).astype(np.float32)


def uniform_offset_scores(m: int, n: int, seed: int) -> np.ndarray:
    """The quantile-balancing demo workload: U(0,1)^{m x n} + U(0,1)^n, fp32."""
    g = _gen(seed, _S_SCORES, 1)
    a = g.random((m, n), dtype=np.float32)
    b = g.random(n, dtype=np.float32)
    return (a + b[None, :]).astype(np.float32)


# ---------------------------------------------------------------- stage inputs
def random_assignment(T: int, N: int, k: int, seed: int, skew: float = 1.0) -> np.ndarray:
    """[T, k] int32 expert ids, distinct per token, drawn with Zipf-like popularity.

    skew = 0 gives uniform popularity; larger skew concentrates tokens on the
    low expert ids (to exercise capacity overflow).
    """
    g = _gen(seed, _S_IDX)
    w = 1.0 / np.arange(1, N + 1, dtype=np.float64) ** skew
    perm = g.permutation(N)
    w = w[perm]
    # Gumbel-top-k sampling without replacement
    gum = -np.log(-np.log(g.random((T, N)))) + np.log(w)[None, :]
    idx = np.argsort(-gum, axis=1, kind="stable")[:, :k]
    return idx.astype(np.int32)


def random_gates(T: int, k: int, seed: int) -> np.ndarray:
    g = _gen(seed, _S_MISC, 1)
    return g.random((T, k), dtype=np.float32)


def random_rows(rows: int, d: int, seed: int, bf16: bool = True) -> np.ndarray:
    g = _gen(seed, _S_MISC, 2)
    y = g.standard_normal((rows, d), dtype=np.float32)
    return bf16_bits(y) if bf16 else y
