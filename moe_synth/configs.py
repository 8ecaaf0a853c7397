"""Workload shapes of the MoE layer forward.

Five workloads, from a tiny fp32 layer to one owner's share of an INT4 expert
pool.  Where they come from:

* tiny fp32: the default MoE of "MoE-Stream" (8 experts, top-2; the
  ``MoEStreamConfig`` dataclass of moe_stream.py) shrunk to d_model 64.
* granular bf16: the MoEEvolve "Architecture" list (d_model 768, 192 SwiGLU
  experts of hidden 256, top-4, one shared expert of hidden 512, capacity-factor
  static-shape dispatch), 16 sequences of the 512-token context.
* wide GeGLU bf16: the kieve-moe "Parametric sizing" flagship (H=768, I=4096,
  E=32, GeGLU experts), top-2, with a Zipf(1.1) per-expert logit bias for skew
  (the additive per-expert logit bias of moe_stream.py ``MoEFFN.forward``).
* decode bf16: the Kvasir "Sharding d'experts" backbone x worker cut (top-8 of
  the softmax, a shared expert, batch 512) at d_model 3072.
* INT4 share: the ExpertMesh Phase-1 profile (896 experts, top-16, packed 4-bit
  weights) as one of 32 stationary owners, d_model 7168, hidden 2048.

``capacity`` is the per-expert pair limit (0 = unlimited).  ``owner``/``owners``
select a round-robin expert share: owner o holds global experts e with
e % owners == o, local id e // owners.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    d: int                 # d_model
    E: int                 # global experts
    k: int                 # top-k
    h: int                 # expert hidden width
    act: str               # "swiglu" | "geglu"
    dtype: str             # activation / dense weight dtype: "f32" | "bf16"
    w_dtype: str           # expert weight dtype: "f32" | "bf16" | "i4g128"
    renorm: bool           # gates renormalised over the k selected
    capacity_factor: Optional[float] = None
    h_shared: int = 0      # 0 = no shared expert
    zipf_bias: Optional[float] = None      # router logit bias -a*ln(e+1)
    logits_input: Optional[float] = None   # Zipf exponent of Gumbel-top-k logits (no router GEMM)
    owners: int = 1        # round-robin expert owners; the share of owner 0 is computed
    seed: int = 0

    @property
    def E_loc(self) -> int:
        return len(range(0, self.E, self.owners))

    @property
    def capacity(self) -> int:
        if self.capacity_factor is None:
            return 0
        return int(math.ceil(self.capacity_factor * self.T * self.k / self.E))

    @property
    def has_router(self) -> bool:
        return self.logits_input is None

    def local_experts(self):
        """Global ids of the experts owned by owner 0, ascending."""
        return list(range(0, self.E, self.owners))


CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=256, d=64, E=8, k=2, h=128, act="swiglu",
                           dtype="f32", w_dtype="f32", renorm=True),
    "granular_bf16": MoEConfig("granular_bf16", T=8192, d=768, E=192, k=4, h=256, act="swiglu",
                               dtype="bf16", w_dtype="bf16", renorm=True, capacity_factor=1.25,
                               h_shared=512),
    "wide_geglu_bf16": MoEConfig("wide_geglu_bf16", T=16384, d=768, E=32, k=2, h=4096,
                                 act="geglu", dtype="bf16", w_dtype="bf16", renorm=True,
                                 zipf_bias=1.1),
    "decode_bf16": MoEConfig("decode_bf16", T=512, d=3072, E=128, k=8, h=768, act="swiglu",
                             dtype="bf16", w_dtype="bf16", renorm=False, h_shared=768),
    "int4_share": MoEConfig("int4_share", T=512, d=7168, E=896, k=16, h=2048, act="swiglu",
                            dtype="bf16", w_dtype="i4g128", renorm=True, logits_input=1.0,
                            owners=32),
}

# Order in which the workloads are listed (tiny first).
WORKLOADS = ["tiny_fp32", "granular_bf16", "wide_geglu_bf16", "decode_bf16", "int4_share"]


@dataclasses.dataclass(frozen=True)
class TreeRouteConfig:
    """Shape of a hierarchical (expert-tree) routing step: T tokens of width d
    routed to k of E experts, the leaves of a tree with ``branch`` children per
    node and ``levels`` levels (kieve-moe "Features", fractal tiling routing)."""
    name: str
    T: int
    d: int
    E: int
    k: int
    branch: int
    levels: int
    dtype: str       # "f32" | "bf16": x and the gate rows
    renorm: bool
    seed: int = 0


# The 896-expert pool of the INT4 share (512 tokens of width 7168, top-16) as a
# 32-ary tree of two levels (28 inner nodes), and a pool of 32,768 experts
# (a 32-ary tree of three levels) at the width of the flagship's larger sibling.
TREE_CONFIGS = {
    "tree_route_896": TreeRouteConfig("tree_route_896", T=512, d=7168, E=896, k=16, branch=32, levels=2,
                                      dtype="bf16", renorm=True),
    "tree_route_32k": TreeRouteConfig("tree_route_32k", T=8192, d=2048, E=32768, k=8, branch=32, levels=3,
                                      dtype="bf16", renorm=True),
}


def config_by_name(name: str) -> MoEConfig:
    return CONFIGS[name]


def scaled(name: str, **over) -> MoEConfig:
    """A copy of a workload with some fields replaced (for small test cases)."""
    base = CONFIGS[name]
    fields = dataclasses.asdict(base)
    fields.update(over)
    if "name" not in over:
        fields["name"] = base.name + "_scaled"
    return MoEConfig(**fields)
