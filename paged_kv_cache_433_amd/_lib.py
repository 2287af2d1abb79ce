"""ctypes loader for libpa.so. Loads on first use and raises if it is missing:
there is no fallback path."""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_UNSUPPORTED = -3
PA_ERR_WORKSPACE = -4
PA_ERR_HIP = -5
PA_DTYPE_BF16 = 0
PA_SWAP_OUT = 0
PA_SWAP_IN = 1
PA_NOALLOC_SCRATCH_BYTES = 17301504

# Every function include/pa.h declares.
EXPORTS = ("pa_decode", "pa_decode_workspace_bytes", "pa_decode_noalloc",
           "pa_decode_step", "pa_decode_step_workspace_bytes",
           "pa_decode_multi", "pa_decode_multi_workspace_bytes",
           "pa_decode_shared", "pa_decode_shared_workspace_bytes",
           "pa_decode_shared_tree", "pa_decode_shared_tree_workspace_bytes",
           "pa_share_plan", "pa_share_plan_bytes", "pa_decode_shared_planned",
           "pa_decode_shared_planned_workspace_bytes",
           "pa_reshape_and_cache", "pa_copy_blocks",
           "pa_swap_blocks", "pa_last_error", "pa_probe_copy", "pa_probe_read", "pa_probe_read_sink_bytes")


class KVCacheDesc(ctypes.Structure):
    """Mirror of ``pa_kv_cache`` in include/pa.h."""

    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def _declare(lib):
    P = ctypes.c_void_p
    I32, I64, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(KVCacheDesc)
    lib.pa_decode.argtypes = [D, P, P, P, I32, I32, I32, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_step.argtypes = [D, P, P, P, P, P, I32, I32, I32, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode_step.restype = ctypes.c_int
    lib.pa_decode_step_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.pa_decode_step_workspace_bytes.restype = SZ
    lib.pa_decode_noalloc.argtypes = [D, P, P, P, I32, I32, I32, ctypes.c_float, P, P]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.pa_decode_workspace_bytes.restype = SZ
    lib.pa_decode_multi.argtypes = [D, P, P, P, I32, I32, I32, I32, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_bytes.argtypes = [D, I32, I32, I32, I32]
    lib.pa_decode_multi_workspace_bytes.restype = SZ
    lib.pa_decode_shared.argtypes = [D, P, P, P, I32, I32, I32, P, P, I32, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode_shared.restype = ctypes.c_int
    lib.pa_decode_shared_workspace_bytes.argtypes = [D, I32, I32, I32, I32]
    lib.pa_decode_shared_workspace_bytes.restype = SZ
    lib.pa_decode_shared_tree.argtypes = [D, P, P, P, I32, I32, I32, P, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode_shared_tree.restype = ctypes.c_int
    lib.pa_decode_shared_tree_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.pa_decode_shared_tree_workspace_bytes.restype = SZ
    lib.pa_share_plan.argtypes = [D, P, I32, I32, I32, P, P, I32, P, P, SZ, P]
    lib.pa_share_plan.restype = ctypes.c_int
    lib.pa_share_plan_bytes.argtypes = [D, I32, I32, I32]
    lib.pa_share_plan_bytes.restype = SZ
    lib.pa_decode_shared_planned.argtypes = [D, P, P, I32, I32, I32, P, ctypes.c_float, P, P, SZ, P]
    lib.pa_decode_shared_planned.restype = ctypes.c_int
    lib.pa_decode_shared_planned_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.pa_decode_shared_planned_workspace_bytes.restype = SZ
    lib.pa_reshape_and_cache.argtypes = [D, P, P, P, I32, P]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [D, P, I32, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_swap_blocks.argtypes = [D, P, P, I64, P, I32, I32, P]
    lib.pa_swap_blocks.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_probe_copy.argtypes = [P, P, SZ, P]
    lib.pa_probe_copy.restype = ctypes.c_int
    lib.pa_probe_read.argtypes = [P, SZ, P, SZ, P]
    lib.pa_probe_read.restype = ctypes.c_int
    lib.pa_probe_read_sink_bytes.argtypes = []
    lib.pa_probe_read_sink_bytes.restype = SZ
    return lib


def lib():
    """The loaded library (raises RuntimeError when it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m paged_kv_cache_433_amd.build` (hipcc, gfx950)")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def last_error() -> str:
    return lib().pa_last_error().decode()
