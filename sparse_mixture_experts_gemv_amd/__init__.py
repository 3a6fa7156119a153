"""Dropless sparse-MoE forward for AMD MI355X (gfx950): hand-written HIP
kernels behind a C ABI (include/moe.h), called through a thin ctypes binding.

    moe_route_topk       router top-k + softmax
    moe_sparse_map       per-expert histogram, exclusive scan, stable route -> slot map
    moe_scatter_ffn_fwd  gathered SwiGLU experts + router-weighted combine (ordered per-route
                         rows by default, fp32 atomic scatter-add with atomic=True)
    moe_scatter_ffn_bwd  its backward: dx, dW1, dW3, dW2 and the router-weight gradient
                         (moe_scatter_ffn_fwd(..., saved=buf) keeps the activations it needs)
    moe_parallel_linear_fwd / moe_parallel_linear_bwd
                         the general ParallelLinear(X, W, I, G) primitive (grouped or scattered
                         input and output) and its backward (dx, dw, dgates)
"""
from ._lib import (MoEError, MoELayer, layer_fwd, load, profile_start, profile_stop, moe_parallel_linear_bwd,
                   moe_parallel_linear_fwd, moe_route_topk, moe_scatter_ffn_bwd, moe_scatter_ffn_fwd, moe_sparse_map,
                   moe_sparse_map_noalloc,
                   parallel_linear_workspace_bytes, route_workspace_bytes, saved_activations_numel,
                   scatter_ffn_bwd_workspace_bytes, scatter_ffn_workspace_bytes, sparse_map_workspace_bytes, status_str)

__all__ = ["MoEError", "MoELayer", "layer_fwd", "load", "profile_start", "profile_stop", "moe_parallel_linear_bwd",
           "moe_parallel_linear_fwd", "moe_route_topk", "moe_scatter_ffn_bwd", "moe_scatter_ffn_fwd", "moe_sparse_map",
           "moe_sparse_map_noalloc", "parallel_linear_workspace_bytes", "route_workspace_bytes", "saved_activations_numel",
           "scatter_ffn_bwd_workspace_bytes",
           "scatter_ffn_workspace_bytes", "sparse_map_workspace_bytes", "status_str"]
