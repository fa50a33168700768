"""ctypes loader for libmoe_int8.so and its C ABI (include/moe_int8.h).

Loading fails loudly when the shared library has not been built: there is no
fallback implementation of any call.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_int8.so")

ABI_VERSION = 6
MOE_OK = 0
STATUS_NAMES = {
    0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE", 4: "MOE_ERR_ALIGN",
    5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_UNSUPPORTED", 7: "MOE_ERR_HIP",
    8: "MOE_ERR_CHECK",
}
MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED = 0, 1, 2
MOE_W_INT8, MOE_W_BF16, MOE_W_FP8 = 0, 1, 2

# every symbol the header declares
EXPORTS = (
    "moe_abi_version", "moe_status_str", "moe_last_error", "moe_workspace_size", "moe_ffn_workspace_size",
    "moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down", "moe_combine", "moe_forward", "moe_quantize_rows",
    "moe_pack_rows", "moe_mlp_workspace_size", "moe_mlp_forward", "moe_quantize_rows_fp8", "moe_down_workspace_size",
    "moe_forward_noalloc", "moe_gate_up_workspace_size", "moe_quantize_pack_rows",
)


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("f", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("ffn_path", ctypes.c_int32), ("weight_fmt", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_SHAPE = ctypes.POINTER(MoeShape)
_SIGS = {
    "moe_abi_version": (ctypes.c_int32, []),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_size": (ctypes.c_int32, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_ffn_workspace_size": (ctypes.c_int32, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P]),
    "moe_permute": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_gate_up": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_gate_up_workspace_size": (ctypes.c_int32, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_expert_down": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_down_workspace_size": (ctypes.c_int32, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_combine": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_quantize_rows": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P]),
    "moe_quantize_rows_fp8": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P]),
    "moe_pack_rows": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "moe_quantize_pack_rows": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                ctypes.c_int32, _P, _P, _P]),
    "moe_mlp_workspace_size": (ctypes.c_int32, [_SHAPE, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_mlp_forward": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_forward_noalloc": (ctypes.c_int32, [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe_int8.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first (python -m int8_weight_moe_amd.build). "
            "There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"libmoe_int8 ABI version {lib.moe_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, _lib.moe_last_error().decode())
