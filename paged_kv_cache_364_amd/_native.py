"""ctypes binding of libpagedkv.so (argument marshalling only).

The library is loaded on first use; a missing library is an error, never a
silent fallback: every operation of this package runs in the HIP kernels or
the C++ allocator of that library.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

c_int = ctypes.c_int
c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_float = ctypes.c_float
vp = ctypes.c_void_p
i32p = ctypes.POINTER(ctypes.c_int32)
i64p = ctypes.POINTER(ctypes.c_int64)
intp = ctypes.POINTER(ctypes.c_int)

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_ALIGN = -3
PKV_ERR_NO_BLOCKS = -4
PKV_ERR_STATE = -5
PKV_ERR_HIP = -6
PKV_ERR_WORKSPACE = -7

DTYPE_F32 = 0
DTYPE_BF16 = 1


class PkvStats(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_free", ctypes.c_int32),
        ("num_used", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_shared", ctypes.c_int32),
        ("logical_tokens", ctypes.c_int64),
        ("table_slots", ctypes.c_int64),
    ]


# name -> (restype, argtypes); the full list of symbols include/pagedkv.h declares
SIGNATURES = {
    "pkv_abi_version": (c_int, []),
    "pkv_status_string": (ctypes.c_char_p, [c_int]),
    "pkv_kv_write": (c_int, [vp, vp, vp, c_int, vp, vp, c_int, c_int, c_int, c_int, c_int, vp]),
    "pkv_copy_blocks": (c_int, [vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp]),
    "pkv_swap_out": (c_int, [vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp]),
    "pkv_swap_in": (c_int, [vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp]),
    "pkv_decode_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "pkv_paged_attention_decode": (c_int, [vp, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, c_int,
                                           c_int, c_float, c_int, vp, c_size, vp]),
    "pkv_paged_attention_decode_append": (c_int, [vp, vp, vp, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, c_int,
                                                  c_int, c_int, c_float, c_int, vp, c_size, vp]),
    "pkv_paged_attention_decode_window": (c_int, [vp, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, c_int,
                                                  c_int, c_int, c_float, c_int, vp, c_size, vp]),
    "pkv_paged_attention_decode_noalloc": (c_int, [vp, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, c_int,
                                                   c_int, c_int, c_float, c_int, vp]),
    "pkv_paged_attention_prefill": (c_int, [vp, vp, vp, c_int, c_int, vp, vp, vp, c_int, vp, c_int, c_int, c_int,
                                            c_int, c_int, c_int, c_float, c_int, vp]),
    "pkv_gather_units": (c_int, [vp, vp, vp, c_int, c_int, c_i64, vp, c_int, vp]),
    "pkv_paged_attention_decode_shared": (c_int, [vp, vp, vp, vp, vp, c_int, vp, c_int, vp, vp, c_int, c_int, c_int,
                                                  c_int, c_int, c_int, c_float, c_int, vp]),
    "pkv_decode_shared_max_members": (c_int, [c_int, c_int]),
    "pkv_shared_prefix_groups": (c_int, [vp, i64p, c_int, c_int, i32p, i32p, intp]),
    "pkv_alloc_create": (vp, [c_int, c_int, i32p]),
    "pkv_alloc_destroy": (None, [vp]),
    "pkv_seq_add": (c_int, [vp, c_i64]),
    "pkv_seq_append": (c_int, [vp, c_i64, c_int, i32p, i32p, c_int, intp]),
    "pkv_seq_append_tokens": (c_int, [vp, c_i64, i32p, c_int, i32p, intp, i32p, c_int, intp]),
    "pkv_prefix_cache_size": (c_int, [vp, intp]),
    "pkv_seq_trim": (c_int, [vp, c_i64, c_i64, intp]),
    "pkv_seq_fork": (c_int, [vp, c_i64, c_i64, c_int]),
    "pkv_seq_free": (c_int, [vp, c_i64]),
    "pkv_seq_swap_out": (c_int, [vp, c_i64, i32p, c_int, intp]),
    "pkv_seq_swap_in": (c_int, [vp, c_i64, i32p, c_int, intp]),
    "pkv_seq_len": (c_int, [vp, c_i64, i64p]),
    "pkv_get_block_table": (c_int, [vp, c_i64, i32p, c_int, intp]),
    "pkv_build_block_tables": (c_int, [vp, i64p, c_int, c_int, i32p, i32p]),
    "pkv_alloc_stats": (c_int, [vp, ctypes.POINTER(PkvStats)]),
    "pkv_block_ref": (c_int, [vp, c_int, intp]),
    "pkv_free_list": (c_int, [vp, i32p, c_int, intp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_364_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib().pkv_status_string(status).decode()
        super().__init__(f"{what}: {msg} ({status})" if what else f"{msg} ({status})")


def check(status: int, what: str = "") -> None:
    if status != PKV_OK:
        raise PagedKVError(status, what)
