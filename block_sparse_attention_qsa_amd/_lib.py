"""ctypes loader for libqsa.so (the HIP library) and its C declarations.

The library is built in-tree (block_sparse_attention_qsa_amd/libqsa.so) by
build.py.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QSA_LIB", os.path.join(_HERE, "libqsa.so"))

QSA_OK = 0
QSA_ERR_INVALID_ARGUMENT = 1
QSA_ERR_UNSUPPORTED = 2
QSA_ERR_WORKSPACE = 3
QSA_ERR_HIP = 4

QSA_KV_BF16 = 0
QSA_KV_FP8_E4M3 = 1
QSA_MAX_SEQ_LEN = 4 * (1 << 21)
QSA_RING_SIZE = 8
QSA_OUT_F32 = 0
QSA_OUT_BF16 = 1


class qsa_config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("compress_ratio", ctypes.c_int32),
        ("topk_blocks", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("ring_size", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_CFG = ctypes.POINTER(qsa_config)

# name -> (restype, argtypes); mirrors include/qsa.h
SIGNATURES = {
    "qsa_ckey_cache_bytes": (ctypes.c_size_t, [_CFG, ctypes.c_int64]),
    "qsa_compress": (_I, [_CFG, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "qsa_index_topk_workspace_size": (ctypes.c_size_t, [_CFG, _I, _I]),
    "qsa_index_topk_workspace_init": (_I, [_P, ctypes.c_size_t, _P]),
    "qsa_index_topk": (_I, [_CFG, _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qsa_index_topk_noalloc": (_I, [_CFG, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "qsa_compress_index_topk": (_I, [_CFG, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]),
    "qsa_prefill_index_topk": (_I, [_CFG, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qsa_sparse_decode": (_I, [_CFG, _I, _I, _I, _I] + [_P] * 14),
    "qsa_select_sparse_decode": (_I, [_CFG, _I, _I, _I, _I, _I] + [_P] * 14 + [ctypes.c_size_t, _P]),
    "qsa_select_sparse_decode_launches": (_I, [_CFG, _I, _I, _I, _I]),
    "qsa_merge_partials": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "qsa_indexer_project_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "qsa_indexer_project": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                 _P, _P, _P, ctypes.c_size_t, _P]),
    "qsa_indexer_project_mrope": (_I, [_I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "qsa_status_string": (ctypes.c_char_p, [_I]),
    "qsa_last_error": (ctypes.c_char_p, []),
    "qsa_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = None) -> ctypes.CDLL:
    """Load libqsa.so once and bind the signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libqsa.so not found at {p}; build it with "
                           "`python -m block_sparse_attention_qsa_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib
