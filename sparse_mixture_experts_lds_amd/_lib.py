"""ctypes view of libmoe_lds.so (declarations mirror include/moe_lds.h)."""
import ctypes
import os

from .build import LIB_PATH

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_I4G128 = 0, 1, 2
MOE_SWIGLU, MOE_GEGLU = 0, 1
MOE_PLACE_ROUND_ROBIN, MOE_PLACE_CONTIGUOUS = 0, 1

# every symbol the header declares
EXPORTS = [
    "moe_route", "moe_router_stats_workspace_bytes", "moe_router_stats", "moe_tree_gate_rows",
    "moe_route_tree_workspace_bytes", "moe_route_tree", "moe_permute_workspace_bytes",
    "moe_permute", "moe_permute_noalloc", "moe_dispatch_owners_workspace_bytes", "moe_dispatch_owners",
    "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_combine", "moe_layer_workspace_bytes", "moe_layer_plan",
    "moe_layer_fwd",
    "moe_layer_bwd_workspace_bytes", "moe_layer_bwd", "moe_quantize_int4", "moe_strerror", "moe_last_error",
]

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("T", _c_int), ("d", _c_int), ("E", _c_int), ("k", _c_int), ("h", _c_int),
        ("act", _c_int), ("act_dtype", _c_int), ("w_dtype", _c_int), ("renorm", _c_int),
        ("capacity", _c_int), ("E_loc", _c_int),
        ("expert_map", _vp), ("w_router", _vp), ("expert_bias", _vp),
        ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp),
        ("s_gate", _vp), ("s_up", _vp), ("s_down", _vp),
        ("h_shared", _c_int),
        ("ws_gate", _vp), ("ws_up", _vp), ("ws_down", _vp),
        ("tile_m", _c_int), ("tile_n_up", _c_int), ("tile_n_down", _c_int),
    ]


MOE_NUM_EVENTS = 7
EVENT_NAMES = ["start", "routed", "grouped", "gate_up", "down", "shared", "end"]


class LayerTrace(ctypes.Structure):
    _fields_ = [("logits", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("expert_offsets", _vp),
                ("pair_pos", _vp), ("events", _vp * MOE_NUM_EVENTS),
                ("expert_counts", _vp), ("prob_mean", _vp), ("balance_loss", _vp),
                ("gate_up_kernel_events", _vp * 2), ("down_kernel_events", _vp * 2)]


class LayerPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("tile_m", "tile_n_up", "tile_n_down", "shared_tile_m",
                                            "shared_in_routed_launches")]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("dx", "dlogits", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down",
                                   "dws_gate", "dws_up", "dws_down", "dgates")]


_LIB = None


def load(path: str = LIB_PATH):
    """Load the library once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            "libmoe_lds.so is not built (%s); run __graft_entry__.build() or "
            "python sparse_mixture_experts_lds_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    sig = {
        "moe_route": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_int,
                               _vp, _vp, _vp, _vp]),
        "moe_router_stats_workspace_bytes": (_c_size, [_c_int, _c_int]),
        "moe_router_stats": (_c_int, [_c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size,
                                      _vp]),
        "moe_tree_gate_rows": (ctypes.c_longlong, [_c_int, _c_int, _c_int]),
        "moe_route_tree_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
        "moe_route_tree": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int,
                                    _vp, _vp, _vp, _c_size, _vp]),
        "moe_permute_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
        "moe_permute": (_c_int, [_c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp,
                                 _vp, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
        "moe_permute_noalloc": (_c_int, [_c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp,
                                         _vp, _c_int, _c_int, _vp, _vp]),
        "moe_dispatch_owners_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
        "moe_dispatch_owners": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
        "moe_expert_ffn_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
        "moe_expert_ffn": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
        "moe_combine": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp]),
        "moe_layer_workspace_bytes": (_c_size, [ctypes.POINTER(LayerDesc)]),
        "moe_layer_plan": (_c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerPlanInfo)]),
        "moe_layer_fwd": (_c_int, [ctypes.POINTER(LayerDesc), _vp, _vp, _vp, ctypes.POINTER(LayerTrace),
                                   _vp, _c_size, _vp]),
        "moe_layer_bwd_workspace_bytes": (_c_size, [ctypes.POINTER(LayerDesc)]),
        "moe_layer_bwd": (_c_int, [ctypes.POINTER(LayerDesc), _vp, _vp, _vp, ctypes.c_float,
                                   ctypes.POINTER(LayerGrads), _vp, _c_size, _vp]),
        "moe_quantize_int4": (_c_int, [_c_int, _c_int, _vp, _vp, _vp, _vp]),
        "moe_strerror": (ctypes.c_char_p, [_c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


class MoEError(RuntimeError):
    def __init__(self, fn: str, code: int):
        lib = load()
        msg = lib.moe_strerror(code).decode()
        if code == MOE_EHIP:
            msg += ": " + lib.moe_last_error().decode()
        super().__init__("%s failed (%d): %s" % (fn, code, msg))
        self.code = code


def check(fn: str, code: int):
    if code != MOE_OK:
        raise MoEError(fn, code)
