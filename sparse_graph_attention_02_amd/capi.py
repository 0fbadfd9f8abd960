"""ctypes binding of libgraph_attn.so (declared in include/graph_attn.h).

The functions here carry the C names and signatures unchanged; each raises
``GraphAttnError`` on a non-OK status instead of returning it.  The library is loaded on
first use and a missing build is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_double, c_float, c_int32, c_int64,
                    c_size_t, c_uint64, c_void_p)

# GRAPH_ATTN_LIB selects another build of the same library (tuning variants).
LIB_PATH = os.environ.get("GRAPH_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libgraph_attn.so")

GA_OK, GA_ERR_INVALID_ARG, GA_ERR_BAD_GRAPH, GA_ERR_UNSUPPORTED = 0, 1, 2, 3
GA_ERR_WORKSPACE, GA_ERR_NOT_READY, GA_ERR_HIP, GA_ERR_HOST_ALLOC = 4, 5, 6, 7
GA_ERR_TOO_LARGE = 8
# bytes of the fixed scratch of graph_attn_fwd_noalloc (GA_FWD_NOALLOC_SCRATCH_BYTES)
GA_FWD_NOALLOC_SCRATCH_BYTES = 64 << 20
GA_F32, GA_BF16 = 0, 1
GA_SCORE_DOT, GA_SCORE_GAT = 0, 1
GA_REDUCE_MAX, GA_REDUCE_MIN = 0, 1


class ga_plan_opts(Structure):
    _fields_ = [("light_max_deg", c_int32), ("hub_min_deg_exclusive", c_int32),
                ("hub_chunk", c_int32), ("build_csc", c_int32), ("feature_slices", c_int32),
                ("col_hub_min_deg_exclusive", c_int32), ("col_hub_chunk", c_int32),
                ("xcd_split_min_deg_exclusive", c_int32),
                ("col_xcd_split_min_deg_exclusive", c_int32)]


class ga_plan_info(Structure):
    _fields_ = [(n, c_int64) for n in (
        "n_nodes", "n_edges", "n_row_light", "n_row_medium", "n_row_hub", "n_row_chunks",
        "has_csc", "n_col_light", "n_col_medium", "n_col_hub", "n_col_chunks",
        "max_in_degree", "max_out_degree", "light_max_deg", "hub_min_deg_exclusive",
        "hub_chunk", "device_bytes", "uploaded", "rows_sorted", "feature_slices",
        "col_hub_min_deg_exclusive", "col_hub_chunk", "xcd_split_min_deg_exclusive",
        "col_xcd_split_min_deg_exclusive", "n_row_sched", "n_col_sched")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class GraphAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)}")


_SIGS = {
    "graph_attn_version": (c_char_p, []),
    "graph_attn_status_string": (c_char_p, [c_int32]),
    "graph_attn_plan_opts_default": (c_int32, [POINTER(ga_plan_opts)]),
    "graph_attn_plan_create": (c_int32, [POINTER(c_int32), POINTER(c_int32), c_int64, c_int64,
                                         POINTER(ga_plan_opts), POINTER(c_void_p)]),
    "graph_attn_plan_get_info": (c_int32, [c_void_p, POINTER(ga_plan_info)]),
    "graph_attn_plan_device_bytes": (c_int32, [c_void_p, POINTER(c_size_t)]),
    "graph_attn_plan_upload": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "graph_attn_plan_array": (c_int32, [c_void_p, c_char_p, POINTER(POINTER(c_int32)),
                                        POINTER(c_int64)]),
    "graph_attn_plan_array_count": (c_int32, []),
    "graph_attn_plan_array_name": (c_char_p, [c_int32]),
    "graph_attn_plan_destroy": (None, [c_void_p]),
    "graph_attn_fwd_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_size_t)]),
    "graph_attn_fwd": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_float, c_float,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_size_t, c_void_p]),
    "graph_attn_fwd_noalloc": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                         c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
    "graph_attn_fwd_gatv2": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_float, c_float,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "graph_attn_bwd_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_size_t)]),
    "graph_attn_bwd": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                 c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "graph_attn_bwd_gatv2_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, c_int32,
                                                       POINTER(c_size_t)]),
    "graph_attn_bwd_gatv2": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_float, c_float,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                       c_void_p]),
    "graph_attn_reduce_fwd_workspace_bytes": (c_int32, [c_void_p, c_int32, POINTER(c_size_t)]),
    "graph_attn_reduce_slot_bytes": (c_int32, [c_void_p, POINTER(c_size_t)]),
    "graph_attn_reduce_fwd": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "graph_attn_reduce_bwd_workspace_bytes": (c_int32, [c_void_p, c_int32, POINTER(c_size_t)]),
    "graph_attn_reduce_bwd": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "graph_attn_timer_enable": (c_int32, [c_int32]),
    "graph_attn_timer_reset": (c_int32, []),
    "graph_attn_timer_count": (c_int32, []),
    "graph_attn_timer_read": (c_int32, [c_int32, POINTER(c_char_p), POINTER(c_int64),
                                        POINTER(c_double)]),
    "graph_attn_copy_probe": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "graph_attn_gather_probe": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p]),
    "graph_attn_gather_probe_cols": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p]),
    "graph_attn_gather_probe_random": (c_int32, [c_int32, c_void_p, c_int64, c_int64, c_uint64,
                                                 c_void_p, c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_graph_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_names():
    return list(_SIGS)


def _status_string(s: int) -> str:
    return lib().graph_attn_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != GA_OK:
        raise GraphAttnError(status, where)


def _wrap(name):
    def call(*args):
        r = getattr(lib(), name)(*args)
        if _SIGS[name][0] is c_int32 and name not in ("graph_attn_plan_array_count",
                                                      "graph_attn_timer_count"):
            _check(r, name)
        return r
    call.__name__ = name
    call.__doc__ = f"ctypes call of `{name}` (include/graph_attn.h); raises GraphAttnError."
    return call


graph_attn_version = _wrap("graph_attn_version")
graph_attn_status_string = _wrap("graph_attn_status_string")
graph_attn_plan_opts_default = _wrap("graph_attn_plan_opts_default")
graph_attn_plan_create = _wrap("graph_attn_plan_create")
graph_attn_plan_get_info = _wrap("graph_attn_plan_get_info")
graph_attn_plan_device_bytes = _wrap("graph_attn_plan_device_bytes")
graph_attn_plan_upload = _wrap("graph_attn_plan_upload")
graph_attn_plan_array = _wrap("graph_attn_plan_array")
graph_attn_plan_array_count = _wrap("graph_attn_plan_array_count")
graph_attn_plan_array_name = _wrap("graph_attn_plan_array_name")
graph_attn_plan_destroy = _wrap("graph_attn_plan_destroy")
graph_attn_fwd_workspace_bytes = _wrap("graph_attn_fwd_workspace_bytes")
graph_attn_fwd = _wrap("graph_attn_fwd")
graph_attn_fwd_noalloc = _wrap("graph_attn_fwd_noalloc")
graph_attn_fwd_gatv2 = _wrap("graph_attn_fwd_gatv2")
graph_attn_bwd_workspace_bytes = _wrap("graph_attn_bwd_workspace_bytes")
graph_attn_bwd = _wrap("graph_attn_bwd")
graph_attn_bwd_gatv2_workspace_bytes = _wrap("graph_attn_bwd_gatv2_workspace_bytes")
graph_attn_bwd_gatv2 = _wrap("graph_attn_bwd_gatv2")
graph_attn_reduce_fwd_workspace_bytes = _wrap("graph_attn_reduce_fwd_workspace_bytes")
graph_attn_reduce_slot_bytes = _wrap("graph_attn_reduce_slot_bytes")
graph_attn_reduce_fwd = _wrap("graph_attn_reduce_fwd")
graph_attn_reduce_bwd_workspace_bytes = _wrap("graph_attn_reduce_bwd_workspace_bytes")
graph_attn_reduce_bwd = _wrap("graph_attn_reduce_bwd")
graph_attn_timer_enable = _wrap("graph_attn_timer_enable")
graph_attn_timer_reset = _wrap("graph_attn_timer_reset")
graph_attn_timer_count = _wrap("graph_attn_timer_count")
graph_attn_timer_read = _wrap("graph_attn_timer_read")
graph_attn_copy_probe = _wrap("graph_attn_copy_probe")
graph_attn_gather_probe = _wrap("graph_attn_gather_probe")
graph_attn_gather_probe_cols = _wrap("graph_attn_gather_probe_cols")
graph_attn_gather_probe_random = _wrap("graph_attn_gather_probe_random")


def raw_status(name: str, *args) -> int:
    """Call a status-returning entry point and return its status instead of raising."""
    return int(getattr(lib(), name)(*args))
