"""ctypes view of ``libmoe.so`` (the C ABI declared in ``include/moe.h``).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names another build of the same library (the host-sanitizer
# build, for instance); by default the in-tree libmoe.so is loaded
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1

MOE_OP_DISPATCH = 1
MOE_OP_EXPERT_FFN = 2
MOE_OP_FORWARD = 3
MOE_OP_BACKWARD = 4
MOE_OP_EXPERT_FFN_FP8 = 5

MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 32
MOE_NO_ALLOC_SCRATCH_BYTES = 1 << 20

# every function the header declares, with its ctypes signature
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", _i32), ("E", _i32), ("k", _i32), ("f", _i32),
                ("dtype", _i32)]


class MoeForwardOutputs(ctypes.Structure):
    _fields_ = [("logits", _p), ("topk_ids", _p), ("topk_gates", _p), ("counts", _p),
                ("offsets", _p), ("sorted_assign", _p), ("assign_pos", _p), ("y_perm", _p)]


class MoeForwardState(ctypes.Structure):
    _fields_ = [("topk_ids", _p), ("topk_gates", _p), ("offsets", _p), ("sorted_assign", _p),
                ("assign_pos", _p), ("y_perm", _p)]


class MoeFp8Weights(ctypes.Structure):
    _fields_ = [("w_gate", _p), ("w_gate_exp", _p), ("w_up", _p), ("w_up_exp", _p), ("w_down", _p),
                ("w_down_exp", _p)]


class MoeBackwardOutputs(ctypes.Structure):
    _fields_ = [("dx", _p), ("dw_gate", _p), ("dw_up", _p), ("dw_down", _p), ("dw_router", _p),
                ("dlogits", _p)]


_PP = ctypes.POINTER(MoeProblem)

SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_abi_version": (_i32, []),
    "moe_workspace_size": (_i32, [_PP, _i32, ctypes.POINTER(_sz)]),
    "moe_route": (_i32, [_PP, _p, _p, _p, _p, _p, _p, _p]),
    "moe_dispatch": (_i32, [_PP, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_dispatch_no_alloc": (_i32, [_PP, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_expert_ffn": (_i32, [_PP, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_combine": (_i32, [_PP, _p, _p, _p, _p, _p]),
    "moe_forward": (_i32, [_PP, _p, _p, _p, _p, _p, _p, _p, ctypes.POINTER(MoeForwardOutputs),
                           _p, _sz, _p]),
    "moe_backward_weights": (_i32, [_PP, _p, _p, _p, _p, _p, _p]),
    "moe_quantize_rows_fp8": (_i32, [_p, ctypes.c_int64, _i32, _p, _p, _p]),
    "moe_mfma_peak": (_i32, [_i32, _i32, _p, _p]),
    "moe_stream_copy": (_i32, [_p, _p, _sz, _p]),
    "moe_quantize_weights_fp8": (_i32, [_PP, _p, _p, _p, ctypes.POINTER(MoeFp8Weights), _p]),
    "moe_expert_ffn_fp8": (_i32, [_PP, _p, _p, _p, ctypes.POINTER(MoeFp8Weights), _p, _p, _sz, _p]),
    "moe_backward": (_i32, [_PP, _p, _p, _p, _p, _p, _p, ctypes.POINTER(MoeForwardState), _p,
                            ctypes.POINTER(MoeBackwardOutputs), _p, _sz, _p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Loads libmoe.so once and attaches the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m mixture_experts_layer_exclusive_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoeError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        name = load().moe_status_string(status).decode()
        super().__init__(f"{where}: {name} ({status})")


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
