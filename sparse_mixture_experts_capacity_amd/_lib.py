"""ctypes view of libmoe.so (include/moe.h).  Loading fails loudly when the
library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16 = 0, 1
TOPK_THEN_SOFTMAX, SOFTMAX_THEN_TOPK = 0, 1
PATH_AUTO, PATH_GROUPED, PATH_STREAM = 0, 1, 2
OVERFLOW_DROP, OVERFLOW_REROUTE, OVERFLOW_SEQUENTIAL = 0, 1, 2
WEIGHTS_ROW_MAJOR, WEIGHTS_PACKED = 0, 1


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("gating", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("dtype", ctypes.c_int32),
        ("ffn_path", ctypes.c_int32),
        ("logit_bias", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("overflow", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
        ("out_fp32", ctypes.c_int32),
    ]


class MoeStats(ctypes.Structure):
    _fields_ = [
        ("capacity", ctypes.c_int64),
        ("assignments", ctypes.c_int64),
        ("dropped", ctypes.c_int64),
        ("counts", ctypes.POINTER(ctypes.c_int64)),
        ("kept", ctypes.POINTER(ctypes.c_int64)),
        ("aux_loss", ctypes.c_double),
        ("aux_loss_kept", ctypes.c_double),
        ("overflow_rate", ctypes.c_double),
        ("entropy_load", ctypes.c_double),
        ("entropy_token", ctypes.c_double),
        ("overflowed", ctypes.c_int64),
        ("rerouted", ctypes.c_int64),
        ("rounds", ctypes.c_int64),
    ]


def _load():
    # PyTorch ships its own HIP runtime (soname libamdhip64.so.7).  Importing
    # torch first makes libmoe's libamdhip64.so.7 dependency bind to that same
    # runtime, so the process holds one HIP/HSA runtime and torch's device
    # memory and streams are valid in the library.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python sparse_mixture_experts_capacity_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    CFG = ctypes.POINTER(MoeConfig)
    ST = ctypes.POINTER(MoeStats)
    sig = {
        "moe_check_config": (ctypes.c_int, [CFG]),
        "moe_workspace_size": (ctypes.c_size_t, [CFG]),
        "moe_capacity": (ctypes.c_int64, [CFG]),
        "moe_forward": (ctypes.c_int, [P, P, P, P, P, CFG, P, ST]),
        "moe_forward_noalloc": (ctypes.c_int, [P, P, P, P, P, CFG, P, ST]),
        "moe_route": (ctypes.c_int, [P, P, CFG, P, P, P, P, P, P, P, ST]),
        "moe_route_logits": (ctypes.c_int, [P, CFG, P, P, P, P, P, P, ST]),
        "moe_aux_loss": (ctypes.c_int, [P, P, CFG, ctypes.POINTER(ctypes.c_double)]),
        "moe_router_backward": (ctypes.c_int, [P, P, P, ctypes.c_double, ctypes.c_double, CFG,
                                               P, P, P, P]),
        "moe_packed_weight_bytes": (ctypes.c_int, [CFG, ctypes.POINTER(ctypes.c_size_t),
                                                   ctypes.POINTER(ctypes.c_size_t)]),
        "moe_pack_weights": (ctypes.c_int, [P, P, P, CFG, P, P, P]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_debug_canaries": (ctypes.c_int, [ctypes.c_int]),
        "moe_debug_check": (ctypes.c_int, [CFG]),
        "moe_entropy_coef": (ctypes.c_double, [ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                               ctypes.c_double]),
        "moe_lb_trend": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]),
        "moe_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "moe_timing_only": (ctypes.c_int, [ctypes.c_char_p]),
        "moe_timing_reset": (ctypes.c_int, []),
        "moe_timing_read": (ctypes.c_int, [ctypes.c_char_p,
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib, tuple(sig)


LIB, EXPORTED_SYMBOLS = _load()
