"""ctypes declarations of the C ABI in include/pa.h (argument marshalling only).

Loading fails loudly when libpa.so has not been built: there is no fallback
path of any kind.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK, PA_ERR_INVALID, PA_ERR_NOMEM, PA_ERR_HIP, PA_ERR_STATE = 0, -1, -2, -3, -4
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)
c_intp = ctypes.POINTER(ctypes.c_int)
c_i64p = ctypes.POINTER(ctypes.c_int64)
c_dblp = ctypes.POINTER(ctypes.c_double)
c_sizep = ctypes.POINTER(ctypes.c_size_t)

# name -> (restype, argtypes); the order of include/pa.h
SIGNATURES = {
    "pa_create_pool": (c_int, [ctypes.POINTER(c_void_p), c_int, c_int, c_int, c_int, c_int, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_int, c_int, c_i32p]),
    "pa_destroy_pool": (c_int, [c_void_p]),
    "pa_alloc_blocks": (c_int, [c_void_p, c_int, c_int, c_int]),
    "pa_set_kv_scales": (c_int, [c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    "pa_append_kv": (c_int, [c_void_p, c_i32p, c_int, c_i32p, c_void_p, c_void_p, c_void_p]),
    "pa_decode": (c_int, [c_void_p, c_i32p, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_int,
                          c_void_p, c_size_t, c_void_p]),
    "pa_decode_noalloc": (c_int, [c_void_p, c_i32p, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_int,
                                  c_void_p]),
    "pa_verify": (c_int, [c_void_p, c_i32p, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p,
                          c_int, c_void_p, c_size_t, c_void_p]),
    "pa_swap_bytes": (c_int, [c_void_p, c_int, ctypes.POINTER(c_size_t)]),
    "pa_swap_out": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_intp, c_void_p]),
    "pa_swap_in": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "pa_prefix_insert": (c_int, [c_void_p, c_int, c_i32p, c_int, c_intp]),
    "pa_prefix_match": (c_int, [c_void_p, c_i32p, c_int, c_intp]),
    "pa_alloc_from_prefix": (c_int, [c_void_p, c_int, c_i32p, c_int, c_intp]),
    "pa_prefix_evict": (c_int, [c_void_p, c_int, c_intp]),
    "pa_prefix_entries": (c_int, [c_void_p, c_intp]),
    "pa_prefill": (c_int, [c_void_p, c_i32p, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p,
                           c_int, c_void_p, c_size_t, c_void_p]),
    "pa_append_attend": (c_int, [c_void_p, c_i32p, c_int, c_int, c_void_p, c_void_p, c_int, c_float, c_void_p,
                                 c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "pa_graph_prepare": (c_int, [c_void_p, c_i32p, c_int, c_int, c_void_p, c_void_p, c_int, c_float, c_void_p,
                                 c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p, c_intp]),
    "pa_graph_launch": (c_int, [c_void_p, c_void_p]),
    "pa_truncate": (c_int, [c_void_p, c_int, c_int]),
    "pa_truncate_batch": (c_int, [c_void_p, c_i32p, c_int, c_i32p]),
    "pa_free_seq": (c_int, [c_void_p, c_int]),
    "pa_sync_tables": (c_int, [c_void_p, c_void_p]),
    "pa_workspace_size": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_sizep]),
    "pa_get_block_table": (c_int, [c_void_p, c_int, c_i32p, c_int, c_intp, c_intp]),
    "pa_get_refcount": (c_int, [c_void_p, c_int, c_intp]),
    "pa_num_free_blocks": (c_int, [c_void_p, c_intp]),
    "pa_last_partition": (c_int, [c_void_p, c_intp, c_intp]),
    "pa_last_call_stats": (c_int, [c_void_p, c_void_p]),
    "pa_get_free_list": (c_int, [c_void_p, c_i32p, c_int, c_intp]),
    "pa_strerror": (ctypes.c_char_p, [c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_profile_enable": (c_int, [c_void_p, c_int]),
    "pa_profile_read": (c_int, [c_void_p, c_int, c_dblp, c_i64p]),
}



class CallStats(ctypes.Structure):
    """pa_call_stats (include/pa.h)."""
    _fields_ = [("partition_tokens", ctypes.c_int32), ("prefix_workgroups", ctypes.c_int32),
                ("attention_workgroups", ctypes.c_int32), ("append_workgroups", ctypes.c_int32),
                ("merge_workgroups", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("prefix_kv_tokens", ctypes.c_int64), ("prefix_query_rows", ctypes.c_int64),
                ("partial_rows", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libpa.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_216_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class PaInvalid(PaError):
    pass


class PaNoMem(PaError):
    pass


class PaHipError(PaError):
    pass


class PaStateError(PaError):
    pass


_ERRORS = {PA_ERR_INVALID: PaInvalid, PA_ERR_NOMEM: PaNoMem, PA_ERR_HIP: PaHipError, PA_ERR_STATE: PaStateError}


def check(code: int) -> None:
    if code == PA_OK:
        return
    lib = load()
    msg = lib.pa_last_error().decode(errors="replace") or lib.pa_strerror(code).decode()
    raise _ERRORS.get(code, PaError)(code, msg)


def i32_array(values):
    vals = [int(v) for v in values]
    arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    return arr, len(vals)
