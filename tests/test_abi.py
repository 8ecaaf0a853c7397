"""The C-ABI library loads, exports every function the header declares, and
rejects bad arguments before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_lds_amd as moe
from sparse_mixture_experts_lds_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe_lds.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = moe.load()
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_texts():
    lib = moe.load()
    for code in (0, -1, -2, -3, -4):
        assert lib.moe_strerror(code)
    assert lib.moe_last_error() == b""


def test_argument_errors_before_launch():
    lib = moe.load()
    P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    # k > E, k = 0, E beyond the limit, d not a multiple of 64
    assert lib.moe_route(4, 64, 8, 9, 0, P, P, None, None, 1, P, P, None, None) == _lib.MOE_EINVAL
    assert lib.moe_route(4, 64, 8, 0, 0, P, P, None, None, 1, P, P, None, None) == _lib.MOE_EINVAL
    assert lib.moe_route(4, 64, 2048, 2, 0, P, P, None, None, 1, P, P, None, None) == _lib.MOE_EUNSUPPORTED
    assert lib.moe_route(4, 65, 8, 2, 0, P, P, None, None, 1, P, P, None, None) == _lib.MOE_EUNSUPPORTED
    assert lib.moe_route(4, 64, 8, 2, 0, None, P, None, None, 1, P, P, None, None) == _lib.MOE_EINVAL
    assert lib.moe_route(4, 64, 8, 2, 7, P, P, None, None, 1, P, P, None, None) == _lib.MOE_EUNSUPPORTED
    # permute: workspace too small, E_loc without a map, negative capacity
    need = lib.moe_permute_workspace_bytes(100, 2, 8)
    assert need > 0
    assert lib.moe_permute(100, 2, 8, P, None, 8, 0, P, P, P, None, 0, 1, None, P, need - 1, None) == _lib.MOE_EWORKSPACE
    assert lib.moe_permute(100, 2, 8, P, None, 4, 0, P, P, P, None, 0, 1, None, P, need, None) == _lib.MOE_EINVAL
    assert lib.moe_permute(100, 2, 8, P, None, 8, -1, P, P, P, None, 0, 1, None, P, need, None) == _lib.MOE_EINVAL
    # the allocation-free grouping: the same checks, and sizes beyond its static
    # scratch (2^22 pairs over 1024 experts: 4096 blocks x 1024 x 4 B = 16 MiB)
    assert lib.moe_permute_noalloc(100, 2, 8, P, None, 4, 0, P, P, P, None, 0, 1, None, None) == _lib.MOE_EINVAL
    assert lib.moe_permute_noalloc(100, 2, 8, P, None, 8, -1, P, P, P, None, 0, 1, None, None) == _lib.MOE_EINVAL
    assert lib.moe_permute_noalloc(1 << 20, 4, 1024, P, None, 1024, 0, P, P, P, None, 0, 1, None,
                                   None) == _lib.MOE_EUNSUPPORTED
    # expert FFN: fp32 activations with bf16 weights; INT4 with d % 128 != 0; missing scales
    nb = lib.moe_expert_ffn_workspace_bytes(4, 64, 256, 128, 1)
    assert lib.moe_expert_ffn(4, 64, 256, 128, 0, 0, 1, P, P, P, P, P, None, None, None, P, P, nb, None) == _lib.MOE_EUNSUPPORTED
    assert lib.moe_expert_ffn(4, 64, 192, 128, 0, 1, 2, P, P, P, P, P, P, P, P, P, P, nb, None) == _lib.MOE_EUNSUPPORTED
    assert lib.moe_expert_ffn(4, 64, 256, 128, 0, 1, 2, P, P, P, P, P, None, P, P, P, P, nb, None) == _lib.MOE_EINVAL
    assert lib.moe_expert_ffn(4, 64, 256, 128, 0, 1, 1, P, P, P, P, P, None, None, None, P, P, nb - 1, None) == _lib.MOE_EWORKSPACE
    assert lib.moe_expert_ffn(4, 64, 256, 128, 5, 1, 1, P, P, P, P, P, None, None, None, P, P, nb, None) == _lib.MOE_EUNSUPPORTED
    # combine: k too large
    assert lib.moe_combine(4, 64, 128, 1, P, P, P, None, P, None) == _lib.MOE_EUNSUPPORTED
    # quantiser: K not a multiple of 128
    assert lib.moe_quantize_int4(4, 200, P, P, P, None) == _lib.MOE_EUNSUPPORTED


def test_misaligned_arrays_rejected_before_launch():
    lib = moe.load()
    # Q is a multiple of 4 bytes, not of 16; R of neither
    P, Q, R = ctypes.c_void_p(16), ctypes.c_void_p(20), ctypes.c_void_p(18)
    assert lib.moe_route(4, 64, 8, 2, 1, Q, P, None, None, 1, P, P, None, None) == _lib.MOE_EINVAL
    assert lib.moe_route(4, 64, 8, 2, 1, P, P, None, None, 1, R, P, None, None) == _lib.MOE_EINVAL
    assert lib.moe_combine(4, 2, 128, 1, Q, P, P, None, P, None) == _lib.MOE_EINVAL
    assert lib.moe_combine(4, 2, 128, 1, P, R, P, None, P, None) == _lib.MOE_EINVAL
    nb = lib.moe_expert_ffn_workspace_bytes(4, 64, 256, 128, 1)
    assert lib.moe_expert_ffn(4, 64, 256, 128, 0, 1, 1, P, P, P, P, Q, None, None, None, P, P, nb, None) == _lib.MOE_EINVAL
    assert lib.moe_quantize_int4(4, 256, P, R, P, None) == _lib.MOE_EINVAL
    nl = lib.moe_layer_workspace_bytes(ctypes.byref(_desc()))
    assert lib.moe_layer_fwd(ctypes.byref(_desc()), Q, None, P, None, P, nl, None) == _lib.MOE_EINVAL
    bad = _desc()
    bad.w_gate = 24
    assert lib.moe_layer_fwd(ctypes.byref(bad), P, None, P, None, P, nl, None) == _lib.MOE_EINVAL


def _desc(**over):
    L = _lib.LayerDesc()
    base = dict(T=64, d=128, E=8, k=2, h=128, act=0, act_dtype=1, w_dtype=1, renorm=1, capacity=0,
                E_loc=8, h_shared=0)
    base.update(over)
    for k, v in base.items():
        setattr(L, k, v)
    L.w_router = L.w_gate = L.w_up = L.w_down = 16
    return L


def test_layer_workspace_and_validation():
    lib = moe.load()
    L = _desc()
    nb = lib.moe_layer_workspace_bytes(ctypes.byref(L))
    assert nb > 64 * 2 * 128 * 2  # at least the expert outputs
    # a bigger T needs more workspace
    assert lib.moe_layer_workspace_bytes(ctypes.byref(_desc(T=640))) > nb
    # shared expert adds its buffers
    Ls = _desc(h_shared=128)
    Ls.ws_gate = Ls.ws_up = Ls.ws_down = 16
    assert lib.moe_layer_workspace_bytes(ctypes.byref(Ls)) > nb
    P = ctypes.c_void_p(16)
    assert lib.moe_layer_fwd(ctypes.byref(L), P, None, P, None, P, nb - 1, None) == _lib.MOE_EWORKSPACE
    bad = _desc(E_loc=4)  # E_loc != E without an expert map
    assert lib.moe_layer_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.moe_layer_fwd(ctypes.byref(bad), P, None, P, None, P, 1 << 30, None) == _lib.MOE_EINVAL
    i4 = _desc(w_dtype=2)  # INT4 without scales
    assert lib.moe_layer_fwd(ctypes.byref(i4), P, None, P, None, P, 1 << 30, None) == _lib.MOE_EINVAL
    f32i4 = _desc(act_dtype=0, w_dtype=2)
    assert lib.moe_layer_fwd(ctypes.byref(f32i4), P, None, P, None, P, 1 << 30, None) == _lib.MOE_EUNSUPPORTED
    # no router weights and no logits
    nr = _desc()
    nr.w_router = None
    assert lib.moe_layer_fwd(ctypes.byref(nr), P, None, P, None, P, 1 << 30, None) == _lib.MOE_EINVAL


@pytest.mark.parametrize("T", [0])
def test_empty_batch_layer_is_a_no_op(T):
    lib = moe.load()
    L = _desc(T=T)
    nb = lib.moe_layer_workspace_bytes(ctypes.byref(L))
    assert lib.moe_layer_fwd(ctypes.byref(L), None, None, None, None, None, nb, None) == _lib.MOE_OK


def _plan(L):
    lib = moe.load()
    info = _lib.LayerPlanInfo()
    rc = lib.moe_layer_plan(ctypes.byref(L), ctypes.byref(info))
    return rc, {n: getattr(info, n) for n, _ in _lib.LayerPlanInfo._fields_}


def _cfg_desc(name, **over):
    from moe_synth import CONFIGS
    c = CONFIGS[name]
    f = dict(T=c.T, d=c.d, E=c.E, k=c.k, h=c.h, act=0 if c.act == "swiglu" else 1,
             act_dtype=0 if c.dtype == "f32" else 1, w_dtype={"f32": 0, "bf16": 1, "i4g128": 2}[c.w_dtype],
             E_loc=c.E, h_shared=c.h_shared)
    f.update(over)
    L = _desc(**f)
    if L.h_shared:
        L.ws_gate = L.ws_up = L.ws_down = 16
    return L


def test_layer_plan():
    # granular: routed and shared GEMMs both on 256-row tiles, in shared launches
    rc, p = _plan(_cfg_desc("granular_bf16"))
    assert rc == _lib.MOE_OK
    assert p == dict(tile_m=256, tile_n_up=128, tile_n_down=256, shared_tile_m=256, shared_in_routed_launches=1)
    # narrow tiles asked for: the shared expert keeps its own launches
    rc, p = _plan(_cfg_desc("granular_bf16", tile_m=128))
    assert rc == _lib.MOE_OK and p["tile_m"] == 128 and p["shared_in_routed_launches"] == 0
    # decode: a few rows per expert, narrow tiles; the shared expert (same
    # hidden width) is the second problem of the routed launches, on their tiles
    rc, p = _plan(_cfg_desc("decode_bf16"))
    assert rc == _lib.MOE_OK and p["tile_m"] < 256 and p["shared_in_routed_launches"] == 1
    assert p["shared_tile_m"] == p["tile_m"]
    # another shared width on narrow tiles: after the routed experts
    rc, p = _plan(_cfg_desc("decode_bf16", h_shared=512))
    assert rc == _lib.MOE_OK and p["tile_m"] < 256 and p["shared_in_routed_launches"] == 0
    # no shared expert
    rc, p = _plan(_cfg_desc("granular_bf16", h_shared=0))
    assert rc == _lib.MOE_OK and p["shared_tile_m"] == 0 and p["shared_in_routed_launches"] == 0
    # fp32 layers never take the wide kernel
    rc, p = _plan(_cfg_desc("tiny_fp32"))
    assert rc == _lib.MOE_OK and p["tile_m"] <= 32 and p["shared_in_routed_launches"] == 0
    # rejected as the workspace query rejects it; no output struct is an error
    rc, _ = _plan(_desc(E_loc=4))
    assert rc == _lib.MOE_EINVAL
    assert moe.load().moe_layer_plan(ctypes.byref(_desc()), None) == _lib.MOE_EINVAL


def test_layer_workspace_covers_router_slices():
    # 512 tokens x 3072 inputs x 128 experts: the router splits its inputs into
    # 8 slices whose partial logits the workspace holds next to the rest
    lib = moe.load()
    L = _cfg_desc("decode_bf16")
    nb = lib.moe_layer_workspace_bytes(ctypes.byref(L))
    assert nb >= 8 * 512 * 128 * 4
    # without a router (logits given) no logits buffer is needed at all
    L2 = _cfg_desc("decode_bf16")
    L2.w_router = None
    assert lib.moe_layer_workspace_bytes(ctypes.byref(L2)) <= nb - 8 * 512 * 128 * 4


def test_tree_router_shape_queries_and_argument_errors():
    import oracle as orc
    lib = moe.load()
    # gate rows of the expert tree: one per non-root node (trimmed trees too)
    for E, B, L in ((896, 32, 2), (32768, 32, 3), (20, 3, 3), (16, 2, 4), (8, 8, 1), (5, 8, 1), (1, 2, 3)):
        assert moe.tree_gate_rows(E, B, L) == orc.tree_nodes(E, B, L)[1][L]
    assert lib.moe_tree_gate_rows(9, 2, 3) == _lib.MOE_EUNSUPPORTED      # E > B^L
    assert lib.moe_tree_gate_rows(8, 1, 3) == _lib.MOE_EUNSUPPORTED      # branch 1
    assert lib.moe_tree_gate_rows(8, 65, 1) == _lib.MOE_EUNSUPPORTED     # branch past 64
    assert lib.moe_tree_gate_rows(8, 2, 0) == _lib.MOE_EINVAL
    P = ctypes.c_void_p(16)  # never dereferenced
    need = lib.moe_route_tree_workspace_bytes(100, 64, 896, 16, 32, 2, 1)
    assert need > 0

    def call(T=100, d=64, E=896, k=16, B=32, L=2, dt=1, x=P, w=P, ids=P, tw=P, ws=P, nb=need):
        return lib.moe_route_tree(T, d, E, k, B, L, dt, x, w, 1, ids, tw, ws, nb, None)

    assert call(nb=need - 1) == _lib.MOE_EWORKSPACE
    assert call(k=0) == _lib.MOE_EINVAL and call(E=8, k=9, B=8, L=1) == _lib.MOE_EINVAL
    assert call(d=96) == _lib.MOE_EUNSUPPORTED                       # d not a multiple of 64
    assert call(k=33) == _lib.MOE_EUNSUPPORTED                       # k past 32
    assert call(k=32, B=64, E=4096) == _lib.MOE_EUNSUPPORTED         # k * branch past 1024
    assert call(E=1025 * 2, B=2, L=12) == _lib.MOE_EUNSUPPORTED      # 1025 nodes above the leaves
    assert call(E=2000, B=32, L=2) == _lib.MOE_EUNSUPPORTED          # E > B^L
    assert call(dt=2) == _lib.MOE_EUNSUPPORTED                       # INT4 activations
    assert call(x=None) == _lib.MOE_EINVAL and call(ws=None) == _lib.MOE_EINVAL
    # T = 0 is a no-op that needs no buffers
    assert lib.moe_route_tree(0, 64, 896, 16, 32, 2, 1, None, None, 1, None, None, None, 0, None) == _lib.MOE_OK
