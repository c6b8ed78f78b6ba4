"""MI355X-native MoE routing, load-balance and dispatch path.

The compute lives in libmoe.so (HIP kernels for gfx950 behind the C ABI of
include/moe.h); this package is its Python binding.  There is no CPU
fallback: every call needs the built library and a GPU.
"""
from .api import (MoeError, allocate_layer_outputs, balance_duals, balance_duals_minibatch,  # noqa: F401
                  balance_signsgd, capacity, combine, dispatch, dispatch_rows, expert_ffn, global_aux,
                  global_aux_hybrid, pack_expert_weights, route, route_lossfree, route_noalloc, router_prepare, shape,
                  stats, switch_layer, switch_layer_backward, workspace_size)
from ._lib import LIB_PATH, load  # noqa: F401

__all__ = ["route", "route_lossfree", "route_noalloc", "router_prepare", "stats", "global_aux", "global_aux_hybrid", "balance_duals",
           "balance_duals_minibatch", "balance_signsgd", "dispatch", "dispatch_rows", "expert_ffn", "pack_expert_weights", "combine",
           "switch_layer", "switch_layer_backward", "capacity", "MoeError", "load", "LIB_PATH"]
