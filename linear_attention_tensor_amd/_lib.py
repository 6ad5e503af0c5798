"""ctypes loader for libtc.so (the C ABI declared in include/tc.h).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtc.so")

TC_OK, TC_ERR_INVALID_ARG, TC_ERR_UNSUPPORTED, TC_ERR_WORKSPACE, TC_ERR_HIP, TC_ERR_INTERNAL = range(6)
TC_F32, TC_BF16 = 0, 1
STATUS_NAMES = {
    TC_OK: "TC_OK",
    TC_ERR_INVALID_ARG: "TC_ERR_INVALID_ARG",
    TC_ERR_UNSUPPORTED: "TC_ERR_UNSUPPORTED",
    TC_ERR_WORKSPACE: "TC_ERR_WORKSPACE",
    TC_ERR_HIP: "TC_ERR_HIP",
    TC_ERR_INTERNAL: "TC_ERR_INTERNAL",
}
SIZE_MAX = ctypes.c_size_t(-1).value

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_z = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tc.h
SIGNATURES = {
    "tc_scan_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "tc_scan_forward": (_i, [_p, _p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _z, _p]),
    "tc_scan_forward_noalloc": (_i, [_p, _p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "tc_scan_backward_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "tc_scan_backward": (_i, [_p, _p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p,
                              _p, _p, _p, _z, _p]),
    "tc_decode_step": (_i, [_p, _p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "tc_decode_layer_step": (_i, [_p, _p, _p, _i, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p,
                                  _p]),
    "tc_fused_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "tc_fused_layer": (_i, [_p, _p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _z, _p]),
    "tc_window_attention": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p]),
    "tc_window_attention_backward_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i]),
    "tc_window_attention_backward": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _z, _p]),
    "tc_fused_layer_backward_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "tc_fused_layer_backward": (_i, [_p, _p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p,
                                     _p, _p, _p, _z, _p]),
    "delta_scan_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i]),
    "delta_scan_forward": (_i, [_p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _z, _p]),
    "delta_scan_backward_workspace_bytes": (_z, [_i, _i, _i, _i, _i, _i, _i]),
    "delta_scan_backward": (_i, [_p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                 _z, _p]),
    "hebbian_workspace_bytes": (_z, [_i, _i, _i]),
    "hebbian_write": (_i, [_p, _p, _p, _i, _i, _p, _p, _i, _i, _p, _p, _z, _p]),
    "hebbian_read": (_i, [_p, _i, _p, _p, _p, _i, _i, _p, _p]),
    "tc_memory_read": (_i, [_p, _p, _i, _i, _i, _p, _p]),
    "recall_argmax": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p]),
    "tc_profile_next_call": (_i, [_p, _p]),
    "tc_last_error": (ctypes.c_char_p, []),
    "tc_version": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class TCError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m linear_attention_tensor_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(L, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = L
    return _lib


def last_error() -> str:
    return lib().tc_last_error().decode()


def check(fn: str, status: int) -> None:
    if status != TC_OK:
        raise TCError(fn, status, last_error())
