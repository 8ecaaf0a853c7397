"""CPU oracle for the top-k routed MoE FFN layer forward.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU product path never routes through it, and it shares no code
with the HIP library (no kernels, headers, helpers, tables or constants).

Everything is float64 NumPy; inputs are read after rounding to their storage
dtype and upcast exactly.  See ``moe_oracle`` for the function list and the
passages each function follows.
"""
from .moe_oracle import (  # noqa: F401
    router_logits, select_topk, gates, route, router_stats, placement, owner_dispatch, permute, silu, gelu_erf, gated_ffn,
    quantize_int4, dequantize_int4, pack_int4, unpack_int4, round_to_dtype,
    moe_layer, LayerWeights, combine, act_grad, gated_ffn_bwd, moe_layer_bwd,
    tree_nodes, tree_route, tree_path_logprob,
)
