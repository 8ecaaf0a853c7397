"""Seeded input generation for the MoE layer forward.

Recipe.  Two PCG64 streams: ``default_rng(seed)`` for the dense inputs and
``default_rng([seed, 1])`` for the routed expert weights, so that the routing of
a workload does not depend on how its expert weights were drawn.  Every normal
is drawn as float64, scaled by its standard deviation (1/sqrt(fan_in)), then
cast to float32.  Dense stream, in this order:

1. activations x ``[T, d]`` ~ N(0, 1);
2. router weights ``[E, d]`` ~ N(0, 1/sqrt(d)) (absent when logits are an input);
3. the shared expert's gate, up ``[h_s, d]`` ~ N(0, 1/sqrt(d)) and down ``[d, h_s]``
   ~ N(0, 1/sqrt(h_s));
4. logits-as-input workloads only: Gumbel(0, 1) noise ``G [T, E]``; the logits
   are ``G[t, e] - a*ln(e + 1)`` (Gumbel-top-k sampling of k experts without
   replacement from a Zipf(a) popularity law).

Expert stream: for each local expert in ascending global id, gate ``[h, d]`` and
up ``[h, d]`` ~ N(0, 1/sqrt(d)), then down ``[d, h]`` ~ N(0, 1/sqrt(h)).

bf16 workloads round the float32 draws to bf16 (round-to-nearest-even, torch).
The per-expert router bias of skewed workloads is ``-a*ln(e + 1)`` in float32.
INT4 workloads keep float32 expert weights here; quantising them is the
caller's business (it is part of the method, not of input generation).

``fast_weights=True`` draws the expert weights with a seeded torch generator
instead (on the given device); used for timing runs of the largest workloads,
where only the distribution matters.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float64) * sigma).astype(np.float32)


def _to_dtype(a: np.ndarray, dt: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "f32":
        return t
    return t.to(torch.bfloat16)


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor                      # [T, d] activation dtype
    w_router: Optional[torch.Tensor]     # [E, d] activation dtype, or None
    bias: Optional[torch.Tensor]         # [E] float32, or None
    logits: Optional[torch.Tensor]       # [T, E] float32, or None
    wg: torch.Tensor                     # [E_loc, h, d] (float32 before quantisation for INT4)
    wu: torch.Tensor                     # [E_loc, h, d]
    wd: torch.Tensor                     # [E_loc, d, h]
    wsg: Optional[torch.Tensor]          # [h_s, d] or None
    wsu: Optional[torch.Tensor]
    wsd: Optional[torch.Tensor]          # [d, h_s]
    expert_map: Optional[np.ndarray]     # [E] int32: global id -> local id or -1; None = identity
    capacity: int

    @property
    def E_loc(self) -> int:
        return self.cfg.E_loc


def expert_map_round_robin(E: int, owners: int, owner: int = 0) -> np.ndarray:
    m = np.full(E, -1, dtype=np.int32)
    mine = np.arange(owner, E, owners)
    m[mine] = np.arange(len(mine), dtype=np.int32)
    return m


def make_inputs(cfg: MoEConfig, fast_weights: bool = False, device: str = "cpu") -> MoEInputs:
    rng = np.random.default_rng(cfg.seed)
    rng_exp = np.random.default_rng([cfg.seed, 1])
    T, d, E, h = cfg.T, cfg.d, cfg.E, cfg.h
    x = _to_dtype(_normal(rng, (T, d), 1.0), cfg.dtype)
    w_router = None
    if cfg.has_router:
        w_router = _to_dtype(_normal(rng, (E, d), 1.0 / np.sqrt(d)), cfg.dtype)
    wdt = "f32" if cfg.w_dtype in ("f32", "i4g128") else "bf16"
    n_loc = cfg.E_loc
    if fast_weights:
        g = torch.Generator(device=device)
        g.manual_seed(cfg.seed + 1)

        def draw(shape, sigma):
            t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma
            return t if wdt == "f32" else t.to(torch.bfloat16)

        wg = draw((n_loc, h, d), 1.0 / np.sqrt(d))
        wu = draw((n_loc, h, d), 1.0 / np.sqrt(d))
        wd = draw((n_loc, d, h), 1.0 / np.sqrt(h))
    else:
        wg = torch.empty((n_loc, h, d), dtype=_TORCH_DT[wdt])
        wu = torch.empty((n_loc, h, d), dtype=_TORCH_DT[wdt])
        wd = torch.empty((n_loc, d, h), dtype=_TORCH_DT[wdt])
        for i in range(n_loc):
            wg[i] = _to_dtype(_normal(rng_exp, (h, d), 1.0 / np.sqrt(d)), wdt)
            wu[i] = _to_dtype(_normal(rng_exp, (h, d), 1.0 / np.sqrt(d)), wdt)
            wd[i] = _to_dtype(_normal(rng_exp, (d, h), 1.0 / np.sqrt(h)), wdt)
    wsg = wsu = wsd = None
    if cfg.h_shared:
        hs = cfg.h_shared
        wsg = _to_dtype(_normal(rng, (hs, d), 1.0 / np.sqrt(d)), cfg.dtype)
        wsu = _to_dtype(_normal(rng, (hs, d), 1.0 / np.sqrt(d)), cfg.dtype)
        wsd = _to_dtype(_normal(rng, (d, hs), 1.0 / np.sqrt(hs)), cfg.dtype)
    logits = None
    if cfg.logits_input is not None:
        gum = rng.gumbel(0.0, 1.0, size=(T, E))
        logits = torch.from_numpy((gum - cfg.logits_input * np.log1p(np.arange(E, dtype=np.float64)))
                                  .astype(np.float32))
    bias = None
    if cfg.zipf_bias is not None:
        bias = torch.from_numpy((-cfg.zipf_bias * np.log1p(np.arange(E, dtype=np.float64)))
                                .astype(np.float32))
    emap = expert_map_round_robin(E, cfg.owners) if cfg.owners > 1 else None
    return MoEInputs(cfg=cfg, x=x, w_router=w_router, bias=bias, logits=logits, wg=wg, wu=wu,
                     wd=wd, wsg=wsg, wsu=wsu, wsd=wsd, expert_map=emap, capacity=cfg.capacity)


def make_tree_inputs(cfg, rows: int):
    """Inputs of a hierarchical routing step: x ``[T, d]`` ~ N(0, 1), then the
    ``rows`` gate rows ``[rows, d]`` ~ N(0, 1/sqrt(d)), from ``default_rng(seed)``
    in that order, cast to the config's dtype.  The row count is the caller's
    (it follows from the tree's shape, which is the method's business)."""
    rng = np.random.default_rng(cfg.seed)
    x = _to_dtype(_normal(rng, (cfg.T, cfg.d), 1.0), cfg.dtype)
    w = _to_dtype(_normal(rng, (rows, cfg.d), 1.0 / np.sqrt(cfg.d)), cfg.dtype)
    return x, w


def as_f64(t) -> Optional[np.ndarray]:
    """Exact float64 copy of a float32/bf16 tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()
