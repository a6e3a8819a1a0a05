"""ctypes declarations of the C ABI in include/tree_attn.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

# TREE_ATTN_LIB names another build of the same library (the host-sanitized
# build of the CPU tests); by default the in-tree libtree_attn.so.
_LIB_PATH = os.environ.get("TREE_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libtree_attn.so")

TA_OK, TA_EINVAL, TA_ENOMEM, TA_EHIP, TA_EUNSUPPORTED = range(5)
TA_F32, TA_BF16 = 0, 1
STATUS_NAMES = {0: "TA_OK", 1: "TA_EINVAL", 2: "TA_ENOMEM", 3: "TA_EHIP", 4: "TA_EUNSUPPORTED"}

TABLE_IDS = {
    "params": 0, "edges": 1, "nq": 2, "lcum": 3, "groups": 4, "group_qs": 5, "group_vis": 6,
    "chunks": 7, "items": 8, "q_slot_ptr": 9, "q_slots": 10, "runs": 11, "chunk_run_ptr": 12,
    "bfs": 13, "seg_tok": 14, "group_seg": 15, "update_counts": 16, "device_tables": 17,
}
TABLE_COLS = {"groups": 8, "chunks": 3, "items": 5, "runs": 3}

EXPORTED_SYMBOLS = [
    "tree_attn_plan", "tree_attn_decode", "tree_attn_plan_info", "tree_attn_plan_export",
    "tree_attn_timing_enable", "tree_attn_timing_read", "tree_attn_plan_destroy",
    "tree_attn_last_error", "tree_attn_plan_extend", "tree_attn_kv_append", "tree_attn_plan_extend_append",
    "tree_attn_decode_noalloc",
]


class PlanOpts(ctypes.Structure):
    _fields_ = [
        ("ts_q", ctypes.c_int32), ("ts_c", ctypes.c_int32), ("gamma", ctypes.c_int32),
        ("rb", ctypes.c_int32), ("waves", ctypes.c_int32), ("floor_f", ctypes.c_int32),
        ("ncu", ctypes.c_int32), ("no_split", ctypes.c_int32),
        ("force_edges", ctypes.POINTER(ctypes.c_int8)), ("host_only", ctypes.c_int32),
        ("scale", ctypes.c_float), ("poison_workspace", ctypes.c_int32),
        ("stream_rows", ctypes.c_int32),
        ("split_align", ctypes.c_int32), ("no_tile_join", ctypes.c_int32),
        ("fail_alloc_after", ctypes.c_int32), ("force_staging", ctypes.c_int32),
    ]


class PagedKV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int64),
        ("stride_page", ctypes.c_int64), ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
    ]


class TreeAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libtree_attn.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m tree_structured_shared_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.tree_attn_plan.argtypes = [i32p, ctypes.c_int32, i32p, i32p, i32p, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.POINTER(PlanOpts), ctypes.POINTER(ctypes.c_void_p)]
    L.tree_attn_plan.restype = ctypes.c_int
    L.tree_attn_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(PagedKV),
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.tree_attn_decode.restype = ctypes.c_int
    L.tree_attn_decode_noalloc.argtypes = L.tree_attn_decode.argtypes
    L.tree_attn_decode_noalloc.restype = ctypes.c_int
    # leaf_add and new_pages are passed as addresses (int32 arrays)
    L.tree_attn_plan_extend.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p, i32p]
    L.tree_attn_plan_extend.restype = ctypes.c_int
    L.tree_attn_kv_append.argtypes = [ctypes.POINTER(PagedKV), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.tree_attn_kv_append.restype = ctypes.c_int
    L.tree_attn_plan_extend_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.POINTER(PagedKV), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, i32p]
    L.tree_attn_plan_extend_append.restype = ctypes.c_int
    L.tree_attn_plan_info.argtypes = [ctypes.c_void_p, i32p, ctypes.POINTER(ctypes.c_int64), i32p]
    L.tree_attn_plan_info.restype = ctypes.c_int
    L.tree_attn_plan_export.argtypes = [ctypes.c_void_p, ctypes.c_int32, i32p,
                                        ctypes.POINTER(ctypes.c_int64)]
    L.tree_attn_plan_export.restype = ctypes.c_int
    L.tree_attn_timing_enable.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    L.tree_attn_timing_enable.restype = ctypes.c_int
    L.tree_attn_timing_read.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_float), i32p]
    L.tree_attn_timing_read.restype = ctypes.c_int
    L.tree_attn_plan_destroy.argtypes = [ctypes.c_void_p]
    L.tree_attn_plan_destroy.restype = None
    L.tree_attn_last_error.argtypes = []
    L.tree_attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status):
    if status != TA_OK:
        msg = lib().tree_attn_last_error().decode(errors="replace")
        raise TreeAttnError(status, msg)
