"""ctypes binding of libdflash_attn.so (the C ABI in include/dflash_block_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  There is no fallback -- if the library is not
built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash_attn.so")
# the same library built with per-workgroup timeline stamps (a measurement aid)
TIMELINE_LIB_PATH = os.path.join(_HERE, "libdflash_attn_timeline.so")

DFLASH_OK = 0
DFLASH_ERR_INVALID_ARGUMENT = 1
DFLASH_ERR_UNSUPPORTED = 2
DFLASH_ERR_WORKSPACE_TOO_SMALL = 3
DFLASH_ERR_HIP = 4

DFLASH_MERGE_AUTO = 0
DFLASH_MERGE_COMBINE_KERNEL = 1
DFLASH_MERGE_IN_KERNEL = 2

DFLASH_KERNEL_AUTO = 0
DFLASH_KERNEL_REFERENCE = 1
DFLASH_KERNEL_MFMA = 2


class dflash_batch_desc(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_block_len", ctypes.c_int32),
        ("total_kv_len", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("kernel", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("event_attn_begin", ctypes.c_void_p),
        ("event_attn_end", ctypes.c_void_p),
        ("merge_mode", ctypes.c_int32),
    ]


class dflash_plan_info(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("tile_keys", ctypes.c_int32),
        ("rows_per_unit", ctypes.c_int32),
        ("head_dim_padded", ctypes.c_int32),
        ("combine_workgroups", ctypes.c_int32),
        ("merge_in_kernel", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once; raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is not built; run `python -m non_causal_block_amd.build` "
                      "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.dflash_block_attn.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, i32, ctypes.c_float, P, P,
                                      ctypes.POINTER(dflash_batch_desc)]
    lib.dflash_block_attn.restype = ctypes.c_int
    lib.dflash_block_attn_noalloc.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, i32, ctypes.c_float, P, P,
                                              ctypes.POINTER(dflash_batch_desc)]
    lib.dflash_block_attn_noalloc.restype = ctypes.c_int
    lib.dflash_noalloc_scratch_bytes.argtypes = []
    lib.dflash_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.dflash_block_attn_spans.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P, P, i32, i32, ctypes.c_float, P,
                                            P, ctypes.POINTER(dflash_batch_desc)]
    lib.dflash_block_attn_spans.restype = ctypes.c_int
    lib.dflash_block_attn_workspace_size.argtypes = [ctypes.POINTER(dflash_batch_desc), i32, i32, i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.dflash_block_attn_workspace_size.restype = ctypes.c_int
    lib.dflash_block_attn_plan.argtypes = [ctypes.POINTER(dflash_batch_desc), i32, i32, i32,
                                           ctypes.POINTER(dflash_plan_info)]
    lib.dflash_block_attn_plan.restype = ctypes.c_int
    lib.dflash_block_attn_supports.argtypes = [i32, i32, i32]
    lib.dflash_block_attn_supports.restype = ctypes.c_int
    lib.dflash_status_string.argtypes = [ctypes.c_int]
    lib.dflash_status_string.restype = ctypes.c_char_p
    lib.dflash_last_error_message.argtypes = []
    lib.dflash_last_error_message.restype = ctypes.c_char_p
    lib.dflash_abi_version.argtypes = []
    lib.dflash_abi_version.restype = ctypes.c_int
    lib.dflash_block_kv_append.argtypes = [P, P, P, P, P, P, P, i32, i32, P, ctypes.POINTER(dflash_batch_desc)]
    lib.dflash_block_kv_append.restype = ctypes.c_int
    lib.dflash_block_attn_append.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, P, i32, ctypes.c_float, P, P,
                                             ctypes.POINTER(dflash_batch_desc)]
    lib.dflash_block_attn_append.restype = ctypes.c_int
    lib.dflash_block_conv.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, P]
    lib.dflash_block_conv.restype = ctypes.c_int
    lib.dflash_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.dflash_stream_read.restype = ctypes.c_int
    lib.dflash_set_debug_checks.argtypes = [ctypes.c_int]
    lib.dflash_set_debug_checks.restype = ctypes.c_int
    lib.dflash_debug_checks_result.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32)]
    lib.dflash_debug_checks_result.restype = ctypes.c_int
    if hasattr(lib, "dflash_timeline_set_buffer"):  # the timeline build only
        lib.dflash_timeline_set_buffer.argtypes = [P, ctypes.c_size_t]
        lib.dflash_timeline_set_buffer.restype = ctypes.c_int
    _lib = lib
    return lib
