"""Python entry points: argument marshalling around the C ABI only."""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_F32, MOE_GEGLU, MOE_I4G128, MOE_SWIGLU, LayerDesc, LayerGrads, LayerPlanInfo,
                   LayerTrace, check, load)

_ACT = {"swiglu": MOE_SWIGLU, "geglu": MOE_GEGLU}


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def route(x: Optional[torch.Tensor], w_router: Optional[torch.Tensor], k: int, renorm: bool,
          logits: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
          want_logits: bool = False):
    """Router step.  Returns (topk_ids int32 [T,k], topk_w float32 [T,k], logits or None)."""
    lib = load()
    if logits is not None:
        T, E = logits.shape
        d, dt, dev = 0, MOE_F32, logits.device
        if x is not None:
            d, dt = x.shape[1], _dt(x)
    else:
        T, d = x.shape
        E = w_router.shape[0]
        dt, dev = _dt(x), x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    lo = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    check("moe_route", lib.moe_route(T, d, E, k, dt, _p(x) if logits is None else None,
                                     _p(w_router) if logits is None else None, _p(logits), _p(bias),
                                     int(bool(renorm)), _p(ids), _p(tw), _p(lo), _stream(dev)))
    return ids, tw, lo


def tree_gate_rows(E: int, branch: int, levels: int) -> int:
    """Rows of the gate table of an expert tree (one per non-root node)."""
    n = load().moe_tree_gate_rows(E, branch, levels)
    check("moe_tree_gate_rows", n if n < 0 else 0)
    return int(n)


def route_tree_workspace_bytes(T: int, d: int, E: int, k: int, branch: int, levels: int,
                               dtype: torch.dtype = torch.bfloat16) -> int:
    dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load().moe_route_tree_workspace_bytes(T, d, E, k, branch, levels, dt))


def route_tree(x: torch.Tensor, w_tree: torch.Tensor, E: int, k: int, branch: int, levels: int, renorm: bool,
               ws: Optional[torch.Tensor] = None, out=None):
    """Hierarchical routing down an expert tree.  Returns (topk_ids int32 [T,k],
    topk_w float32 [T,k]); ``ws`` (bytes) and ``out`` (ids, w) may be given."""
    lib = load()
    T, d = x.shape
    dev = x.device
    ids, tw = out if out is not None else (torch.empty((T, k), dtype=torch.int32, device=dev),
                                            torch.empty((T, k), dtype=torch.float32, device=dev))
    nb = lib.moe_route_tree_workspace_bytes(T, d, E, k, branch, levels, _dt(x))
    if ws is None:
        ws = _ws(nb, dev)
    check("moe_route_tree", lib.moe_route_tree(T, d, E, k, branch, levels, _dt(x), _p(x), _p(w_tree),
                                               int(bool(renorm)), _p(ids), _p(tw), _p(ws), ws.numel(),
                                               _stream(dev)))
    return ids, tw


def router_stats(logits: torch.Tensor, topk_ids: torch.Tensor, bias: Optional[torch.Tensor] = None):
    """Router by-products.  Returns (expert_counts int32 [E], prob_mean float32 [E],
    balance_loss float32 [1])."""
    lib = load()
    T, E = logits.shape
    k = topk_ids.shape[1]
    dev = logits.device
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    pm = torch.empty(E, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    nb = lib.moe_router_stats_workspace_bytes(T, E)
    ws = _ws(nb, dev)
    check("moe_router_stats", lib.moe_router_stats(T, E, k, _p(logits), _p(bias), _p(topk_ids), _p(cnt), _p(pm),
                                                   _p(loss), _p(ws), nb, _stream(dev)))
    return cnt, pm, loss


def permute_workspace_bytes(T: int, k: int, E_loc: int) -> int:
    return load().moe_permute_workspace_bytes(T, k, E_loc)


def permute(topk_ids: torch.Tensor, E: int, E_loc: Optional[int] = None,
            expert_map: Optional[torch.Tensor] = None, capacity: int = 0,
            x: Optional[torch.Tensor] = None):
    """Grouping step.  Returns (expert_offsets [E_loc+1], sorted_pair [T*k], pair_pos [T*k],
    x_perm [T*k, d] or None)."""
    lib = load()
    T, k = topk_ids.shape
    E_loc = E if E_loc is None else E_loc
    dev = topk_ids.device
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    x_perm = None
    d, dt = 0, MOE_BF16
    if x is not None:
        d, dt = x.shape[1], _dt(x)
        x_perm = torch.zeros((T * k, d), dtype=x.dtype, device=dev)
    nb = lib.moe_permute_workspace_bytes(T, k, E_loc)
    ws = _ws(nb, dev)
    check("moe_permute", lib.moe_permute(T, k, E, _p(topk_ids), _p(expert_map), E_loc, capacity,
                                         _p(offsets), _p(sp), _p(pos), _p(x), d, dt, _p(x_perm),
                                         _p(ws), nb, _stream(dev)))
    return offsets, sp, pos, x_perm


def permute_noalloc(topk_ids: torch.Tensor, E: int, E_loc: Optional[int] = None,
                    expert_map: Optional[torch.Tensor] = None, capacity: int = 0,
                    x: Optional[torch.Tensor] = None, out: Optional[tuple] = None):
    """The grouping step without a workspace (moe_permute_noalloc: the library's
    static scratch).  ``out`` may hold preallocated (expert_offsets, sorted_pair,
    pair_pos, x_perm) tensors; then nothing is allocated here either.  Returns
    the same tuple as ``permute``."""
    lib = load()
    T, k = topk_ids.shape
    E_loc = E if E_loc is None else E_loc
    dev = topk_ids.device
    if out is None:
        offsets = torch.empty(E_loc + 1, dtype=torch.int32, device=dev)
        sp = torch.empty(T * k, dtype=torch.int32, device=dev)
        pos = torch.empty(T * k, dtype=torch.int32, device=dev)
        x_perm = torch.zeros((T * k, x.shape[1]), dtype=x.dtype, device=dev) if x is not None else None
    else:
        offsets, sp, pos, x_perm = out
    d, dt = (x.shape[1], _dt(x)) if x is not None else (0, MOE_BF16)
    check("moe_permute_noalloc", lib.moe_permute_noalloc(T, k, E, _p(topk_ids), _p(expert_map), E_loc, capacity,
                                                         _p(offsets), _p(sp), _p(pos), _p(x), d, dt, _p(x_perm),
                                                         _stream(dev)))
    return offsets, sp, pos, x_perm


_PLACE = {"round_robin": _lib.MOE_PLACE_ROUND_ROBIN, "contiguous": _lib.MOE_PLACE_CONTIGUOUS}


def dispatch_owners(topk_ids: torch.Tensor, E: int, n_owners: int, placement: str = "round_robin",
                    capacity: int = 0, x: Optional[torch.Tensor] = None):
    """Pairs grouped by expert owner (then local expert, then pair index).  Returns a dict
    with owner_offsets [n+1], recv_offsets [n, E/n+1], expert_offsets [E+1], sorted_pair,
    pair_pos [T*k] (int32) and, when x is given, x_send [T*k, d]."""
    lib = load()
    T, k = topk_ids.shape
    dev = topk_ids.device
    i32 = dict(dtype=torch.int32, device=dev)
    r = {"owner_offsets": torch.empty(n_owners + 1, **i32),
         "recv_offsets": torch.empty((n_owners, E // max(n_owners, 1) + 1), **i32),
         "expert_offsets": torch.empty(E + 1, **i32),
         "sorted_pair": torch.empty(max(T * k, 1), **i32),
         "pair_pos": torch.empty(max(T * k, 1), **i32)}
    d, dt = 0, MOE_F32
    if x is not None:
        d, dt = x.shape[1], _dt(x)
        r["x_send"] = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    nb = lib.moe_dispatch_owners_workspace_bytes(T, k, E)
    ws = _ws(nb, dev)
    check("moe_dispatch_owners", lib.moe_dispatch_owners(
        T, k, E, n_owners, _PLACE[placement], int(capacity), _p(topk_ids), _p(r["owner_offsets"]),
        _p(r["recv_offsets"]), _p(r["expert_offsets"]), _p(r["sorted_pair"]), _p(r["pair_pos"]), _p(x), d, dt,
        _p(r.get("x_send")), _p(ws), nb, _stream(dev)))
    return r


def expert_ffn_workspace_bytes(E_loc, rows_max, d, h, act_dtype) -> int:
    return load().moe_expert_ffn_workspace_bytes(E_loc, rows_max, d, h, act_dtype)


def expert_ffn(x_perm: torch.Tensor, offsets: Optional[torch.Tensor], wg, wu, wd, act: str = "swiglu",
               sg=None, su=None, sd=None, w_dtype: Optional[int] = None):
    """Grouped gated FFN over grouped rows.  Weights [E_loc, h, d] / [E_loc, d, h] in the
    activation dtype, or uint8 packed INT4 with float16 scales (sg, su, sd)."""
    lib = load()
    rows, d = x_perm.shape
    dev = x_perm.device
    dt = _dt(x_perm)
    if w_dtype is None:
        w_dtype = MOE_I4G128 if wg.dtype == torch.uint8 else _dt(wg)
    E_loc, h = wg.shape[0], wg.shape[1]
    y = torch.empty((rows, d), dtype=x_perm.dtype, device=dev)
    nb = lib.moe_expert_ffn_workspace_bytes(E_loc, rows, d, h, dt)
    ws = _ws(nb, dev)
    check("moe_expert_ffn", lib.moe_expert_ffn(E_loc, rows, d, h, _ACT[act], dt, w_dtype, _p(x_perm),
                                               _p(offsets), _p(wg), _p(wu), _p(wd), _p(sg), _p(su),
                                               _p(sd), _p(y), _p(ws), nb, _stream(dev)))
    return y


def combine(y_perm: torch.Tensor, pair_pos: torch.Tensor, topk_w: torch.Tensor,
            shared_y: Optional[torch.Tensor] = None):
    """Weighted combine.  topk_w [T, k]; returns out [T, d]."""
    lib = load()
    T, k = topk_w.shape
    d = y_perm.shape[1]
    dev = y_perm.device
    out = torch.empty((T, d), dtype=y_perm.dtype, device=dev)
    check("moe_combine", lib.moe_combine(T, k, d, _dt(y_perm), _p(y_perm), _p(pair_pos), _p(topk_w),
                                         _p(shared_y), _p(out), _stream(dev)))
    return out


def quantize_int4(w: torch.Tensor):
    """float32 [..., N, K] -> (packed uint8 [..., N, K/2], scales float16 [..., N, K/128])."""
    lib = load()
    K = w.shape[-1]
    rows = w.numel() // K
    packed = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (K // 128,), dtype=torch.float16, device=w.device)
    check("moe_quantize_int4", lib.moe_quantize_int4(rows, K, _p(w), _p(packed), _p(scales),
                                                     _stream(w.device)))
    return packed, scales


@dataclasses.dataclass
class LayerWeights:
    """Device tensors of one layer.  wg/wu [E_loc, h, d], wd [E_loc, d, h] in the activation
    dtype, or uint8 packed INT4 (then sg/su/sd hold float16 scales)."""
    E: int
    k: int
    act: str
    renorm: bool
    wg: torch.Tensor
    wu: torch.Tensor
    wd: torch.Tensor
    sg: Optional[torch.Tensor] = None
    su: Optional[torch.Tensor] = None
    sd: Optional[torch.Tensor] = None
    w_router: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    expert_map: Optional[torch.Tensor] = None
    capacity: int = 0
    wsg: Optional[torch.Tensor] = None
    wsu: Optional[torch.Tensor] = None
    wsd: Optional[torch.Tensor] = None
    tiles: tuple = (0, 0, 0)   # (tile_m, tile_n_up, tile_n_down) hints, 0 = automatic

    def desc(self, T: int, d: int, act_dtype: int) -> LayerDesc:
        E_loc, h = self.wg.shape[0], self.wg.shape[1]
        i4 = self.wg.dtype == torch.uint8
        L = LayerDesc()
        L.T, L.d, L.E, L.k, L.h = T, d, self.E, self.k, h
        L.act, L.act_dtype = _ACT[self.act], act_dtype
        L.w_dtype = MOE_I4G128 if i4 else _dt(self.wg)
        L.renorm, L.capacity, L.E_loc = int(bool(self.renorm)), int(self.capacity), E_loc
        for name, t in [("expert_map", self.expert_map), ("w_router", self.w_router),
                        ("expert_bias", self.bias), ("w_gate", self.wg), ("w_up", self.wu),
                        ("w_down", self.wd), ("s_gate", self.sg), ("s_up", self.su),
                        ("s_down", self.sd), ("ws_gate", self.wsg), ("ws_up", self.wsu),
                        ("ws_down", self.wsd)]:
            p = _p(t)
            setattr(L, name, p.value if p is not None else None)
        L.h_shared = self.wsg.shape[0] if self.wsg is not None else 0
        L.tile_m, L.tile_n_up, L.tile_n_down = (int(v) for v in self.tiles)
        return L


def layer_workspace_bytes(weights: LayerWeights, T: int, d: int, act_dtype: int) -> int:
    L = weights.desc(T, d, act_dtype)
    return load().moe_layer_workspace_bytes(ctypes.byref(L))


def layer_plan(weights: LayerWeights, T: int, d: int, act_dtype: int) -> dict:
    """How layer_fwd runs the expert GEMMs for this layer (moe_layer_plan)."""
    L = weights.desc(T, d, act_dtype)
    info = LayerPlanInfo()
    check("moe_layer_plan", load().moe_layer_plan(ctypes.byref(L), ctypes.byref(info)))
    return {n: int(getattr(info, n)) for n, _ in LayerPlanInfo._fields_}


def layer_fwd(x: torch.Tensor, weights: LayerWeights, logits: Optional[torch.Tensor] = None,
              trace: bool = False, out: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None, events=None, stats: bool = False, kernel_events=None):
    """Whole layer forward.  Returns out [T, d] (and a dict of intermediates when trace;
    ``stats`` adds the router by-products expert_counts, prob_mean and balance_loss to it).

    ``events``: optional list of MOE_NUM_EVENTS raw hipEvent_t handles (ints, or None),
    recorded on the current stream at the step boundaries.  ``kernel_events``: optional
    (gate_up_start, gate_up_stop, down_start, down_stop) raw handles attached to the
    routed GEMM launches themselves."""
    lib = load()
    trace = trace or stats
    T, d = x.shape
    dev = x.device
    dt = _dt(x)
    L = weights.desc(T, d, dt)
    nb = lib.moe_layer_workspace_bytes(ctypes.byref(L))
    if nb == 0:
        raise _lib.MoEError("moe_layer_workspace_bytes", _lib.MOE_EINVAL)
    if ws is None or ws.numel() < nb:
        ws = _ws(nb, dev)
    if out is None:
        out = torch.empty((T, d), dtype=x.dtype, device=dev)
    tr = None
    tdict = None
    if events is not None or kernel_events is not None:
        tr = LayerTrace()
        for i, ev in enumerate(events or []):
            tr.events[i] = ev
        if kernel_events is not None:
            tr.gate_up_kernel_events[0], tr.gate_up_kernel_events[1] = kernel_events[0], kernel_events[1]
            tr.down_kernel_events[0], tr.down_kernel_events[1] = kernel_events[2], kernel_events[3]
    if trace:
        E_loc = weights.wg.shape[0]
        k = weights.k
        tdict = {
            "topk_ids": torch.empty((T, k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
            "expert_offsets": torch.empty(E_loc + 1, dtype=torch.int32, device=dev),
            "pair_pos": torch.empty(T * k, dtype=torch.int32, device=dev),
        }
        if logits is None:
            tdict["logits"] = torch.empty((T, weights.E), dtype=torch.float32, device=dev)
        if stats:
            tdict["expert_counts"] = torch.empty(weights.E, dtype=torch.int32, device=dev)
            tdict["prob_mean"] = torch.empty(weights.E, dtype=torch.float32, device=dev)
            tdict["balance_loss"] = torch.empty(1, dtype=torch.float32, device=dev)
        tr = tr if tr is not None else LayerTrace()
        for name, t in tdict.items():
            setattr(tr, name, t.data_ptr())
    check("moe_layer_fwd", lib.moe_layer_fwd(ctypes.byref(L), _p(x), _p(logits), _p(out),
                                             ctypes.byref(tr) if tr is not None else None, _p(ws), nb,
                                             _stream(dev)))
    if trace:
        return out, tdict
    return out


def layer_bwd_workspace_bytes(weights: LayerWeights, T: int, d: int, act_dtype: int) -> int:
    L = weights.desc(T, d, act_dtype)
    return load().moe_layer_bwd_workspace_bytes(ctypes.byref(L))


def layer_bwd(x: torch.Tensor, weights: LayerWeights, dout: torch.Tensor, logits: Optional[torch.Tensor] = None,
              balance: float = 0.0, ws: Optional[torch.Tensor] = None, grads: Optional[dict] = None):
    """Gradients of layer_fwd for the upstream gradient dout (plus balance times the
    balance loss).  Returns a dict: dx, dgates, the weight gradients that exist
    (dw_gate, dw_up, dw_down; dws_* with a shared expert; dw_router with a router;
    dbias with a bias) and dlogits when logits are given.  ``grads`` may hold
    preallocated outputs (a missing key is allocated)."""
    lib = load()
    T, d = x.shape
    dev = x.device
    dt = _dt(x)
    L = weights.desc(T, d, dt)
    nb = lib.moe_layer_bwd_workspace_bytes(ctypes.byref(L))
    if nb == 0:
        raise _lib.MoEError("moe_layer_bwd_workspace_bytes", _lib.MOE_EINVAL)
    if ws is None or ws.numel() < nb:
        ws = _ws(nb, dev)
    E, k = weights.E, weights.k
    E_loc, h = weights.wg.shape[0], weights.wg.shape[1]
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dgates": (T, k), "dw_gate": (E_loc, h, d), "dw_up": (E_loc, h, d), "dw_down": (E_loc, d, h)}
    if weights.wsg is not None:
        hs = weights.wsg.shape[0]
        shapes.update(dws_gate=(hs, d), dws_up=(hs, d), dws_down=(d, hs))
    if weights.w_router is not None and logits is None:
        shapes["dw_router"] = (E, d)
    if weights.bias is not None:
        shapes["dbias"] = (E,)
    if logits is not None:
        shapes["dlogits"] = (T, E)
    out = dict(grads or {})
    if "dx" not in out:
        out["dx"] = torch.empty((T, d), dtype=x.dtype, device=dev)
    for n, shp in shapes.items():
        if n not in out:
            out[n] = torch.empty(shp, **f32)
    g = LayerGrads()
    for n, t in out.items():
        setattr(g, n, t.data_ptr())
    check("moe_layer_bwd", lib.moe_layer_bwd(ctypes.byref(L), _p(x), _p(logits), _p(dout), float(balance),
                                             ctypes.byref(g), _p(ws), nb, _stream(dev)))
    return out
