"""ctypes view of libwkv.so (the C ABI declared in include/wkv.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libwkv.so")

WKV_OK, WKV_ERR_INVALID_ARG, WKV_ERR_UNSUPPORTED, WKV_ERR_DEVICE = 0, 1, 2, 3
WKV_F32, WKV_BF16 = 0, 1
WKV_ALGO_AUTO, WKV_ALGO_SCAN, WKV_ALGO_CHUNKED = 0, 1, 2
WKV_LAYOUT_BTHN, WKV_LAYOUT_BHTN = 0, 1
WKV_DEV_BAD_STATE_MAP = 1
WKV_DEV_BAD_LENGTH = 2
WKV_DEV_TOKEN_OVERFLOW = 4
WKV_DEV_DUPLICATE_ROW = 8

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/wkv.h
SIGNATURES = {
    "wkv4_forward": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp]),
    "wkv4_forward_ex": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp]),
    "wkv5_forward": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp]),
    "wkv5_forward_ex": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _i,
                             _vp, _vp]),
    "wkv6_forward": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp]),
    "wkv6_forward_ex": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _vp, _vp, _i, _vp, _i,
                             _vp, _vp]),
    "wkv7_forward_ex": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _i, _vp,
                             _i, _vp, _vp]),
    "wkv7_forward": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _i, _vp,
                          _vp, _vp]),
    "wkv6_backward": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "wkv6_backward_ex": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp]),
    "wkv6_forward_train": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                                _vp, _vp]),
    "wkv6_backward_noalloc": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "wkv6_forward_varlen": (_i, [_i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i,
                                 _vp, _vp]),
    "wkv6_forward_varlen_ex": (_i, [_i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                                    _vp, _i, _vp, _vp]),
    "wkv_schedule_round_robin": (_i, [_i, _i32p, _i, _i32p, _i32p]),
    "wkv_resolve_algo": (_i, [_i, _i, _i, _i, _i, _i, _i]),
    "wkv_status_string": (ctypes.c_char_p, [_i]),
    "wkv_last_error": (ctypes.c_char_p, []),
    "wkv_abi_version": (_i, []),
}

_lib = None


class WkvError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{detail} [{status_string(status)}]")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libwkv.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libwkv.so not found at {path}; build it with "
            "`python -m rwkv_linear_attention_wkv_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.wkv_abi_version() != 1:
        raise ImportError(f"libwkv.so ABI version {lib.wkv_abi_version()} != 1")
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().wkv_status_string(status).decode()


def check(status: int):
    if status != WKV_OK:
        raise WkvError(status, load().wkv_last_error().decode())
