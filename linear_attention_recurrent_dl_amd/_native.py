"""ctypes view of the C ABI declared in include/deltalog.h.

Argument marshalling only: every function here forwards to the shared library
with the same name.  The library must exist; there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdeltalog.so")

DL_OK = 0
DL_ERR_INVALID_ARG = -1
DL_ERR_UNSUPPORTED = -2
DL_ERR_SLOT_RANGE = -3
DL_ERR_DUPLICATE_SLOT = -4
DL_ERR_BATCH_TOO_LARGE = -5
DL_ERR_HIP = -6
DL_ERR_DRY_RUN = -7

DL_DECAY = {"none": 0, "scalar": 1, "per_key": 2}
DL_UPDATE = {"plain": 0, "delta": 1}
DL_DTYPE = {"f32": 0, "bf16": 1}
DL_NUM_BUFS = 6
BUF_NAMES = ("base", "klog", "ulog", "lamlog", "nlog", "coef")

EXPORTED = ("dl_pool_sizes", "dl_pool_create", "dl_pool_destroy", "dl_slot_assign",
            "dl_decode_step", "dl_eager_step", "dl_merge", "dl_flush_all", "dl_get_log_len",
            "dl_schedule", "dl_read_log_len_device", "dl_value_tile", "dl_last_error",
            "dl_launch_slot_limit", "dl_read_base", "dl_decode_window", "dl_decode_step_noalloc")


class dl_pool_desc(ctypes.Structure):
    _fields_ = [("num_slots", c_int32), ("max_batch", c_int32), ("num_v_heads", c_int32),
                ("num_k_heads", c_int32), ("d_k", c_int32), ("d_v", c_int32),
                ("merge_interval", c_int32), ("decay", c_int32), ("update", c_int32),
                ("state_dtype", c_int32), ("in_dtype", c_int32), ("value_tile", c_int32),
                ("replay_split", c_int32)]


class dl_pool_buffers(ctypes.Structure):
    _fields_ = [("base", c_void_p), ("klog", c_void_p), ("ulog", c_void_p),
                ("lamlog", c_void_p), ("nlog", c_void_p), ("coef", c_void_p)]


class DeltaLogError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} failed ({code}): {msg}")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"DeltaLog HIP library not found at {LIB_PATH}; build it with "
                           "`python -m linear_attention_recurrent_dl_amd.build`")
    # PyTorch ships its own HIP runtime under the same soname; load it first when
    # it is installed so that the library, torch's allocator and torch's streams
    # share one runtime whatever the import order of the caller.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    i32p = POINTER(c_int32)
    sig = {
        "dl_pool_sizes": (c_int, [POINTER(dl_pool_desc), POINTER(c_size_t)]),
        "dl_pool_create": (c_int, [POINTER(dl_pool_desc), POINTER(dl_pool_buffers), POINTER(c_void_p)]),
        "dl_pool_destroy": (c_int, [c_void_p]),
        "dl_slot_assign": (c_int, [c_void_p, c_int32, i32p, c_void_p, c_void_p]),
        "dl_decode_step": (c_int, [c_void_p, c_int32, i32p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p]),
        "dl_eager_step": (c_int, [c_void_p, c_int32, i32p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
        "dl_decode_step_noalloc": (c_int, [c_void_p, c_int32, i32p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_void_p]),
        "dl_decode_window": (c_int, [c_void_p, c_int32, i32p, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p]),
        "dl_merge": (c_int, [c_void_p, c_int32, i32p, c_void_p]),
        "dl_flush_all": (c_int, [c_void_p, c_void_p]),
        "dl_read_base": (c_int, [c_void_p, c_int32, i32p, c_void_p, c_void_p]),
        "dl_get_log_len": (c_int, [c_void_p, i32p]),
        "dl_schedule": (c_int, [c_void_p, c_int32, i32p, i32p, i32p]),
        "dl_read_log_len_device": (c_int, [c_void_p, i32p, c_void_p]),
        "dl_value_tile": (c_int, [POINTER(dl_pool_desc)]),
        "dl_last_error": (c_char_p, []),
        "dl_launch_slot_limit": (c_int32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _LIB = L
    return L


def check(rc: int, func: str) -> None:
    if rc != DL_OK:
        msg = lib().dl_last_error()
        raise DeltaLogError(rc, func, msg.decode() if msg else "")


def ptr(x) -> int:
    """Device or host address of a tensor / array / int (0 for None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(type(x))
