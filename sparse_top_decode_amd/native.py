"""ctypes view of libstdk.so (the C ABI declared in include/stdk.h).

Argument marshalling only: every step of the computation runs in the HIP
library. Loading fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstdk.so")

STDK_OK = 0
STDK_EINVAL = -1
STDK_EUNSUPPORTED = -2
STDK_EWORKSPACE = -3
STDK_EHIP = -4
STDK_F32 = 0
STDK_BF16 = 1
STDK_MAX_RANGES = 16
STDK_NOALLOC_SCRATCH_BYTES = 96 << 20

# every symbol include/stdk.h declares
EXPORTS = [
    "topk_attn_decode", "topk_attn_decode_workspace_size", "attn_merge_lse",
    "topk_attn_decode_static", "topk_attn_decode_static_workspace_size", "topk_attn_decode_static_noalloc",
    "retopk_state_init", "retopk_step", "retopk_step_device", "retopk_workspace_size", "retopk_state_size",
    "topk_multi_query", "topk_multi_query_workspace_size",
    "quantize_keys_int8", "topk_attn_decode_int8", "topk_attn_decode_int8_workspace_size",
    "topk_attn_decode_int8_static", "topk_attn_decode_int8_static_workspace_size",
    "stdk_last_error", "stdk_version", "stdk_inject_launch_failure", "stdk_hbm_read",
    "stdk_profile_enable", "stdk_profile_disable", "stdk_profile_reset", "stdk_profile_read",
]


class Layout(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("max_len", c_int64), ("kv_dtype", c_int32), ("reserved", c_int32),
                ("stride_b", c_int64), ("stride_h", c_int64)]


class RetopkParams(ctypes.Structure):
    _fields_ = [("top_k", c_int32), ("cache_cap", c_int32), ("top_r", c_int32), ("recent", c_int32),
                ("tau", c_float), ("refresh", c_int32), ("scale", c_float), ("budget", c_int32)]


class RetopkState(ctypes.Structure):
    _fields_ = [("q_hat", c_void_p), ("support", c_void_p), ("head", c_void_p), ("count", c_void_p)]


_lib = None


def _sig(lib):
    P = c_void_p
    lib.topk_attn_decode.argtypes = [POINTER(Layout), P, P, P, POINTER(c_int64), c_int32, c_int32, c_float,
                                     P, P, P, P, c_size_t, P]
    lib.topk_attn_decode.restype = c_int32
    lib.topk_attn_decode_workspace_size.argtypes = [POINTER(Layout), c_int64, c_int32]
    lib.topk_attn_decode_workspace_size.restype = c_size_t
    lib.topk_attn_decode_static.argtypes = [POINTER(Layout), P, P, P, POINTER(c_int64), c_int32,
                                            POINTER(c_int64), c_int32, c_int32, c_float, P, P, P, P, c_size_t, P]
    lib.topk_attn_decode_static.restype = c_int32
    lib.topk_attn_decode_static_workspace_size.argtypes = [POINTER(Layout), c_int64, c_int64, c_int32]
    lib.topk_attn_decode_static_workspace_size.restype = c_size_t
    lib.attn_merge_lse.argtypes = [c_int64, c_int32, P, P, P, P, P, P, P]
    lib.attn_merge_lse.restype = c_int32
    lib.topk_attn_decode_static_noalloc.argtypes = [POINTER(Layout), P, P, P, POINTER(c_int64), c_int32,
                                                    POINTER(c_int64), c_int32, c_int32, c_float, P, P, P, P]
    lib.topk_attn_decode_static_noalloc.restype = c_int32
    lib.retopk_state_init.argtypes = [POINTER(Layout), POINTER(RetopkParams), POINTER(RetopkState), P, P, c_int32, P]
    lib.retopk_state_init.restype = c_int32
    lib.retopk_step.argtypes = [POINTER(Layout), POINTER(RetopkParams), POINTER(RetopkState), P, P, P, c_int64,
                                c_int64, P, P, P, P, P, P, P, c_size_t, P]
    lib.retopk_step.restype = c_int32
    lib.retopk_step_device.argtypes = [POINTER(Layout), POINTER(RetopkParams), POINTER(RetopkState), P, P, P, P,
                                       P, P, P, P, P, P, P, c_size_t, P]
    lib.retopk_step_device.restype = c_int32
    lib.topk_multi_query.argtypes = [POINTER(Layout), P, c_int32, P, POINTER(c_int64), c_int32, c_int32, c_float,
                                     P, P, P, c_size_t, P]
    lib.topk_multi_query.restype = c_int32
    lib.topk_multi_query_workspace_size.argtypes = [POINTER(Layout), c_int32, c_int64, c_int32]
    lib.topk_multi_query_workspace_size.restype = c_size_t
    lib.quantize_keys_int8.argtypes = [POINTER(Layout), P, POINTER(c_int64), c_int32, P, P, P]
    lib.quantize_keys_int8.restype = c_int32
    lib.topk_attn_decode_int8.argtypes = [POINTER(Layout), P, P, P, P, P, POINTER(c_int64), c_int32, c_int32, c_int32,
                                          c_float, P, P, P, P, P, c_size_t, P]
    lib.topk_attn_decode_int8.restype = c_int32
    lib.topk_attn_decode_int8_workspace_size.argtypes = [POINTER(Layout), c_int64, c_int32, c_int32]
    lib.topk_attn_decode_int8_workspace_size.restype = c_size_t
    lib.topk_attn_decode_int8_static.argtypes = [POINTER(Layout), P, P, P, P, P, POINTER(c_int64), c_int32,
                                                 POINTER(c_int64), c_int32, c_int32, c_int32, c_float, P, P, P, P,
                                                 P, c_size_t, P]
    lib.topk_attn_decode_int8_static.restype = c_int32
    lib.topk_attn_decode_int8_static_workspace_size.argtypes = [POINTER(Layout), c_int64, c_int64, c_int32, c_int32]
    lib.topk_attn_decode_int8_static_workspace_size.restype = c_size_t
    lib.retopk_workspace_size.argtypes = [POINTER(Layout), POINTER(RetopkParams), c_int64]
    lib.retopk_workspace_size.restype = c_size_t
    lib.retopk_state_size.argtypes = [POINTER(Layout), POINTER(RetopkParams)]
    lib.retopk_state_size.restype = c_size_t
    lib.stdk_hbm_read.argtypes = [P, c_int64, c_int32, c_int64, c_int32, P, P]
    lib.stdk_hbm_read.restype = c_int32
    lib.stdk_inject_launch_failure.argtypes = [c_int32]
    lib.stdk_inject_launch_failure.restype = c_int32
    lib.stdk_last_error.argtypes = []
    lib.stdk_last_error.restype = c_char_p
    lib.stdk_version.argtypes = []
    lib.stdk_version.restype = c_int32
    lib.stdk_profile_enable.argtypes = [c_int32, c_char_p]
    lib.stdk_profile_enable.restype = c_int32
    lib.stdk_profile_disable.argtypes = []
    lib.stdk_profile_disable.restype = c_int32
    lib.stdk_profile_reset.argtypes = []
    lib.stdk_profile_reset.restype = c_int32
    lib.stdk_profile_read.argtypes = [c_char_p, POINTER(c_double), POINTER(c_int64)]
    lib.stdk_profile_read.restype = c_int32


def load():
    """Load libstdk.so (once). Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        _sig(lib)
        _lib = lib
    return _lib


class StdkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"stdk error {code}: {msg}")
        self.code = code


def check(rc: int):
    if rc != STDK_OK:
        raise StdkError(rc, load().stdk_last_error().decode(errors="replace"))
