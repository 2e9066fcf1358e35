"""ctypes loader for libgraft.so (the HIP kernels behind include/graft.h).

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgraft.so")

c_int, c_int64, c_float, c_size_t, c_void_p, c_char_p = (
    ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p)
P = c_void_p  # any pointer (device or host), passed as an integer address

# name -> (restype, argtypes), mirroring include/graft.h
SIGNATURES = {
    "graft_last_error": (c_char_p, []),
    "graft_version": (c_int, []),
    "graft_table_update_retrieve": (c_int, [P, c_int, c_int, c_int, P, P, c_int, P, P,
                                            c_int, P, P, P, P, c_int, P, P, P]),
    "graft_build_tree": (c_int, [c_int, c_int, P, P, P, P, c_int, P, P, P, P, P, P, c_int, c_int,
                                 c_float, P, P, P, P, P, P, P, P, P, P, P]),
    "graft_prune_anchor": (c_int, [c_int, P, P, P, P, c_int, P, P, P, P, P, P]),
    "graft_tree_attention_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "graft_tree_attention": (c_int, [c_int, c_int, c_int, c_int, c_float, P, P, P, P, c_int64,
                                     P, c_int, P, c_int, P, P, P, P, P, c_size_t, P, P]),
    "graft_lmhead_topk_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "graft_lmhead_topk": (c_int, [c_int, c_int, c_int, c_int, P, P, c_int, P, P, P, P, c_size_t, P]),
    "graft_lmhead_pack_bytes": (c_size_t, [c_int, c_int]),
    "graft_lmhead_topk_noalloc_bytes": (c_size_t, [c_int, c_int]),
    "graft_lmhead_topk_noalloc": (c_int, [c_int, c_int, c_int, c_int, P, P, P, P, P]),
    "graft_lmhead_pack": (c_int, [c_int, c_int, P, P, P]),
    "graft_accept": (c_int, [c_int, P, P, P, P, P, c_int, P, P, P, P, P]),
    "graft_lmhead_sample_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "graft_lmhead_topk_sample": (c_int, [c_int, c_int, c_int, c_int, c_float, P, P, P, P, P, P, P, c_size_t, P]),
    "graft_sample_rows": (c_int, [c_int, c_int, c_float, P, P, P, P]),
    "graft_accept_sampled": (c_int, [c_int, P, P, P, P, P, P, P, P, P, P]),
    "graft_treegraft_node_count": (c_int, [c_int, c_int, c_int, c_int]),
    "graft_treegraft_build": (c_int, [c_int, c_int, c_int, c_int, P, P, P, P, P, P, P, P, P, P, P]),
    "graft_tail_cut": (c_int, [c_int, c_int, P, P, P, c_float, P, P, P]),
    "graft_kv_compact": (c_int, [c_int, c_int, c_int, c_int, P, P, c_int64, P, c_int64, P, P, P, P, P, P, P, P,
                                 P]),
    "graft_make_template": (c_int, [c_int, c_int, c_int, P, P]),
    "graft_table_save": (c_int, [c_char_p, c_int, c_int, P, P]),
    "graft_table_load": (c_int, [c_char_p, c_int, c_int, P, P]),
    "graft_stage_budget": (c_int, [c_int, P, P]),
}

GRAFT_OK, GRAFT_EINVAL, GRAFT_EUNSUPPORTED, GRAFT_EHIP, GRAFT_EIO = 0, -1, -2, -3, -4
ERR_TOKEN, ERR_PARENT, ERR_NOT_CLOSED, ERR_CAPACITY, ERR_RANK, ERR_ALIGN = 1, 2, 4, 8, 16, 32
SRC_ROOT, SRC_DRAFT, SRC_RETRIEVED, SRC_REPLACED = 0, 1, 2, 3
TREE_PRUNE, TREE_STATIC_REPLACE, TREE_TAIL = 0, 1, 2
W_ROWMAJOR, W_PACKED = 0, 1
MAX_NODES, MAX_K, MAX_V = 64, 16, (1 << 30) - 1


class GraftError(RuntimeError):
    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m draft_tree_verification_parent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def call(name: str, *args) -> int:
    rc = getattr(lib(), name)(*args)
    if rc != GRAFT_OK:
        raise GraftError(name, rc, lib().graft_last_error().decode())
    return rc
