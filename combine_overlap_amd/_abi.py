"""ctypes view of the C ABI declared in include/moe_overlap.h.

Loading fails loudly (ImportError) when the built library is missing: there
is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_OVERLAP_LIB", os.path.join(_HERE, "libmoe_overlap.so"))

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_TIMEOUT = -5
MOE_ERR_DEVICE = -6
MOE_MAX_RANKS = 16
MOE_GATE_SOFTMAX = 0
MOE_GATE_SIGMOID = 1
MOE_MODE_OVERLAP = 0
MOE_MODE_SEQUENTIAL = 1
MOE_MODE_ROLE_SWITCH = 2
MOE_CONSUMER_AUTO = -1

META_MPAD, META_NBANDS, META_NREMOTE, META_NSEG, META_STATUS, META_NUNITS, META_NTILES, \
    META_NRTILES, META_CAUTO = range(9)
META_PRED = 20   # double over words 20-21


class MoeShape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("R", "T", "H", "F", "E", "k", "r_self", "gated", "gate_kind", "tb_m", "mgb")]


class MoeSizes(C.Structure):
    _fields_ = [("ws_bytes", C.c_size_t), ("m_pad_max", C.c_int64), ("max_bands", C.c_int32),
                ("max_flags", C.c_int32), ("recv_rows_max", C.c_int32), ("bn_out", C.c_int32),
                ("tile_m", C.c_int32), ("max_tiles", C.c_int32)]


PLAN_FIELDS = ("meta", "group_row", "expert_base", "recv_off", "band_row0", "band_expert",
               "band_dest", "band_recv0", "band_valid", "seg_band0", "seg_nbands", "seg_dest",
               "seg_src_row", "seg_dst_row", "seg_rows", "row_src", "recv_row", "chunk_base",
               "chunk_counts", "tile_ctr", "slot_valid", "seg_unit0", "tile_row0", "tile_expert",
               "tile_rows", "tile_sched", "seg_tile0", "seg_tile1", "partial")


class MoePlan(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PLAN_FIELDS]


class MoeCalib(C.Structure):
    _fields_ = [("gemm_flops_per_cu", C.c_double), ("gemm_m_half", C.c_double),
                ("copy_bw_per_cu", C.c_double), ("copy_bw_max", C.c_double),
                ("seg_latency_s", C.c_double), ("n_cu", C.c_int32), ("c_min", C.c_int32),
                ("c_max", C.c_int32), ("c_step", C.c_int32)]


EXPORTS = ("moe_error_string", "moe_query_sizes", "moe_plan_view", "moe_ctx_create",
           "moe_ctx_destroy", "moe_ctx_num_cus", "moe_ctx_set_wait_limit", "moe_ctx_set_debug",
           "moe_ctx_set_timing", "moe_ctx_timings", "moe_ctx_set_trace", "moe_route", "moe_permute",
           "moe_plan_partition", "moe_expert_forward_overlap", "moe_expert_forward_gathered",
           "moe_expert_forward_noalloc",
           "moe_combine", "moe_read_status")

_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with `python combine_overlap_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    vp, i32, u32, pi32 = C.c_void_p, C.c_int32, C.c_uint32, C.POINTER(C.c_int32)
    pshape = C.POINTER(MoeShape)
    L.moe_error_string.restype = C.c_char_p
    L.moe_error_string.argtypes = [C.c_int]
    L.moe_query_sizes.argtypes = [pshape, C.POINTER(MoeSizes)]
    L.moe_plan_view.argtypes = [pshape, vp, C.POINTER(MoePlan)]
    L.moe_ctx_create.argtypes = [C.POINTER(vp)]
    L.moe_ctx_destroy.argtypes = [vp]
    L.moe_ctx_num_cus.argtypes = [vp]
    L.moe_ctx_set_wait_limit.argtypes = [vp, C.c_uint64]
    L.moe_ctx_set_debug.argtypes = [vp, u32, i32, C.c_int64]
    L.moe_ctx_set_timing.argtypes = [vp, C.c_int]
    L.moe_ctx_timings.argtypes = [vp, C.POINTER(C.c_float)]
    L.moe_ctx_set_trace.argtypes = [vp, pshape, vp, C.c_int64]
    L.moe_route.argtypes = [pshape, vp, vp, vp, vp, vp, vp]
    L.moe_permute.argtypes = [pshape, vp, vp, vp, vp, vp, vp]
    L.moe_plan_partition.argtypes = [pshape, pi32, C.POINTER(MoeCalib), pi32, pi32,
                                     C.POINTER(C.c_double)]
    L.moe_expert_forward_overlap.argtypes = [vp, pshape, vp, vp, vp, vp, vp, vp, vp,
                                             C.POINTER(vp), vp, u32, i32, i32, vp]
    L.moe_expert_forward_gathered.argtypes = L.moe_expert_forward_overlap.argtypes
    L.moe_expert_forward_noalloc.argtypes = L.moe_expert_forward_overlap.argtypes
    L.moe_combine.argtypes = [pshape, C.POINTER(vp), vp, vp, vp, vp, vp]
    L.moe_read_status.argtypes = [pshape, vp, pi32, vp]
    for name in EXPORTS:
        if name != "moe_error_string":
            getattr(L, name).restype = C.c_int
    _lib = L
    return L


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({lib().moe_error_string(code).decode()})")
        self.code = code


def check(fn: str, rc: int) -> int:
    if rc != MOE_OK:
        raise MoeError(fn, rc)
    return rc
