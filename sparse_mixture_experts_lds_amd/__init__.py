"""Top-k routed MoE FFN layer forward for AMD MI355X (gfx950).

Thin Python binding of libmoe_lds.so (C ABI in include/moe_lds.h).  Every
function marshals torch CUDA tensors into device pointers, allocates the
outputs and workspace with torch, and passes torch's current HIP stream.  All
arithmetic runs in the library's HIP kernels; nothing here computes.
"""
from .api import (  # noqa: F401
    route, route_tree, route_tree_workspace_bytes, tree_gate_rows, router_stats, permute, permute_noalloc, dispatch_owners, expert_ffn, combine, layer_fwd, quantize_int4, LayerWeights,
    permute_workspace_bytes, expert_ffn_workspace_bytes, layer_workspace_bytes, layer_plan, layer_bwd,
    layer_bwd_workspace_bytes,
)
from ._lib import MoEError, load  # noqa: F401
