"""Seeded synthetic inputs for the top-k routed MoE FFN layer forward.

This package only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no routing, no permutation, no expert math, no quantiser).
Both the CPU oracle and the HIP path are fed from here, and nothing else is
shared between them.
"""
from .configs import CONFIGS, TREE_CONFIGS, WORKLOADS, TreeRouteConfig, scaled, config_by_name  # noqa: F401
from .generate import make_inputs, make_tree_inputs, MoEInputs  # noqa: F401
