"""Helpers for the GPU parity tests: host <-> device conversion and comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_rel(got, ref, rtol, what, floor=0.0):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref) / np.maximum(np.abs(ref), floor if floor > 0 else np.finfo(np.float64).tiny)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rtol, f"{what}: max relative error {worst:.3e} > {rtol:.1e}"
    return worst


def row_rel_err(got, ref):
    """Per-row max |got - ref| / max |ref| (rows of a [T, d] output)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), np.finfo(np.float64).tiny)
    return num / den


def check_selection(gpu_idx, ref, what, rel=1e-6):
    """Bit-exact top-k indices except near-tie tokens (oracle margin < rel); returns the
    set of tokens whose selection differs (all of them near-ties)."""
    gpu_idx = np.asarray(gpu_idx)
    diff = np.nonzero(np.any(gpu_idx != ref.idx, axis=1))[0]
    near = set(ref.near_ties(rel).tolist())
    bad = [int(t) for t in diff if t not in near]
    assert not bad, f"{what}: {len(bad)} tokens differ outside the near-tie set, e.g. {bad[:5]}"
    if len(diff):
        say(f"{what}: {len(diff)} near-tie tokens chose differently (of {len(near)} near ties)")
    return set(int(t) for t in diff)
