"""ctypes declarations of the C ABI in ``include/pa.h``.

Loads ``libpa.so`` from this package directory. There is no fallback: if the
library is missing, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os
import re

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pa.h")

PA_OK = 0
PA_NOALLOC_SCRATCH_BYTES = 16 << 20   # include/pa.h
PA_ERR_NO_BLOCKS = -7
PA_ERR_SEQUENCE = -8
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


class PaKvCache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int),
        ("block_size", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_L = ctypes.c_int64
_CACHE = ctypes.POINTER(PaKvCache)

SIGNATURES = {
    "pa_write_kv": (_I, [_CACHE, _P, _P, _P, _I, _P]),
    "pa_decode": (_I, [_CACHE, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P]),
    "pa_splitk_num_splits": (_I, [_I, _I]),
    "pa_splitk_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "pa_decode_splitk": (_I, [_CACHE, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "pa_lse_merge": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pa_varlen_workspace_bytes": (ctypes.c_size_t, [_CACHE, _I, _I, _I, _I]),
    "pa_varlen": (_I, [_CACHE, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                       ctypes.c_size_t, _P]),
    "pa_status_str": (ctypes.c_char_p, [_I]),
    "pa_decode_balanced_workspace_bytes": (ctypes.c_size_t, [_CACHE, _I, _I]),
    "pa_decode_balanced": (_I, [_CACHE, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, ctypes.c_size_t,
                                _P]),
    "pa_write_decode_balanced": (_I, [_CACHE, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P,
                                      ctypes.c_size_t, _P]),
    "pa_write_decode_balanced_noalloc": (_I, [_CACHE, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                              _F, _P]),
    "pa_copy_blocks": (_I, [_CACHE, _P, _I, _P]),
    "pa_rope_write_kv": (_I, [_CACHE, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "pa_bm_create": (_P, [_I, _I]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_num_free": (_I, [_P]),
    "pa_bm_blocks_needed": (_L, [_P, _L, _L]),
    "pa_bm_append": (_I, [_P, _L, _L, _P]),
    "pa_bm_append_batch": (_I, [_P, _P, _P, _I, _P, _P]),
    "pa_bm_block_tables": (_I, [_P, _P, _I, _P, _I, _P]),
    "pa_bm_fork": (_I, [_P, _L, _L]),
    "pa_bm_free": (_I, [_P, _L]),
    "pa_bm_seq_len": (_L, [_P, _L]),
    "pa_bm_block_table": (_I, [_P, _L, _P, _I]),
    "pa_bm_ref_count": (_I, [_P, _I]),
    "pa_bm_take_copies": (_I, [_P, _P, _I]),
}

_lib = None


def header_symbols() -> list[str]:
    """Names of the functions ``include/pa.h`` declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc for gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
