"""MI355X-native MoE routing, load-balance and dispatch path.

The compute lives in libmoe.so (HIP kernels for gfx950 behind the C ABI of
include/moe.h); this package is its Python binding.  There is no CPU
fallback: every call needs the built library and a GPU.
"""
from .api import (MoeError, balance_duals, balance_signsgd, capacity, combine, dispatch, dispatch_rows, expert_ffn,  # noqa: F401
                  global_aux, global_aux_hybrid, route, router_prepare, stats, switch_layer, workspace_size, allocate_layer_outputs,
                  shape)
from ._lib import LIB_PATH, load  # noqa: F401

__all__ = ["route", "router_prepare", "stats", "global_aux", "global_aux_hybrid", "balance_duals", "balance_signsgd", "dispatch", "dispatch_rows", "expert_ffn", "combine", "switch_layer",
           "capacity", "MoeError", "load", "LIB_PATH"]
