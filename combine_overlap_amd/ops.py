"""Thin Python binding of the C ABI: same names, argument marshalling only.

Tensors are torch device tensors (bf16 tensors carry the bf16 bit patterns
the ABI expects); streams are torch.cuda.Stream objects (None = current).
Every function raises MoeError when the library returns an error code.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np

from . import _abi
from ._abi import MoeCalib, MoePlan, MoeShape, MoeSizes, check, lib


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def make_shape(R, T, H, F, E, k, r_self, gated, gate_kind, tb_m, mgb=1) -> MoeShape:
    gk = gate_kind
    if isinstance(gk, str):
        gk = {"softmax": _abi.MOE_GATE_SOFTMAX, "sigmoid": _abi.MOE_GATE_SIGMOID}[gk]
    return MoeShape(int(R), int(T), int(H), int(F), int(E), int(k), int(r_self), int(bool(gated)),
                    int(gk), int(tb_m), int(mgb))


def moe_query_sizes(shape: MoeShape) -> MoeSizes:
    out = MoeSizes()
    check("moe_query_sizes", lib().moe_query_sizes(C.byref(shape), C.byref(out)))
    return out


def moe_plan_view(shape: MoeShape, ws) -> dict:
    out = MoePlan()
    check("moe_plan_view", lib().moe_plan_view(C.byref(shape), C.c_void_p(_ptr(ws)), C.byref(out)))
    return {n: getattr(out, n) for n in _abi.PLAN_FIELDS}


class Context:
    """Owns a moe_ctx_t (the device's CU count, optional timing events)."""

    def __init__(self):
        h = C.c_void_p()
        check("moe_ctx_create", lib().moe_ctx_create(C.byref(h)))
        self.handle = h
        self.num_cus = lib().moe_ctx_num_cus(h)

    def set_wait_limit(self, ticks: int):
        """Bound on each wait of a copying role for ready flags, in 100 MHz
        ticks (0: the default of 2 s); see moe_ctx_set_wait_limit."""
        check("moe_ctx_set_wait_limit", lib().moe_ctx_set_wait_limit(self.handle, int(ticks)))

    def set_debug(self, delay_seed: int = 0, reverse_schedule: bool = False, tail_wait_ticks: int = -1):
        """Test knobs (timing only; see moe_ctx_set_debug): seeded per-item
        delays, reversed tile queues, the split tail chunks' wait bound."""
        check("moe_ctx_set_debug", lib().moe_ctx_set_debug(self.handle, int(delay_seed) & 0xFFFFFFFF,
                                                           int(bool(reverse_schedule)), int(tail_wait_ticks)))

    def set_timing(self, enable: bool):
        check("moe_ctx_set_timing", lib().moe_ctx_set_timing(self.handle, int(bool(enable))))

    def timings(self) -> dict:
        """Phase times (ms) of the last timed forward; keys as in the header."""
        ms = (C.c_float * 5)()
        check("moe_ctx_timings", lib().moe_ctx_timings(self.handle, ms))
        return dict(gemm1=ms[0], producer=ms[1], producer_start_to_consumer_end=ms[2], total=ms[3],
                    exposed=ms[4])

    def set_trace(self, shape, trace=None):
        """Device timeline buffer (uint64 words; see moe_ctx_set_trace) or None to stop."""
        n = 0 if trace is None else trace.numel()
        check("moe_ctx_set_trace", lib().moe_ctx_set_trace(self.handle, C.byref(shape), _ptr(trace), n))

    def close(self):
        if self.handle:
            check("moe_ctx_destroy", lib().moe_ctx_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_route(shape, logits, topk_ids, gates, counts, ws, stream=None):
    check("moe_route", lib().moe_route(C.byref(shape), _ptr(logits), _ptr(topk_ids), _ptr(gates),
                                       _ptr(counts), _ptr(ws), _stream(stream)))


def moe_permute(shape, x, topk_ids, counts, x_perm, ws, stream=None):
    check("moe_permute", lib().moe_permute(C.byref(shape), _ptr(x), _ptr(topk_ids), _ptr(counts),
                                           _ptr(x_perm), _ptr(ws), _stream(stream)))


def moe_plan_partition(shape, counts_host: np.ndarray, calib: Optional[MoeCalib] = None):
    """Returns (n_consumer_cu, mgb, predicted_seconds); counts_host is [E_l, R] int32."""
    cnt = np.ascontiguousarray(counts_host, dtype=np.int32)
    c, g, t = C.c_int32(), C.c_int32(), C.c_double()
    check("moe_plan_partition", lib().moe_plan_partition(
        C.byref(shape), cnt.ctypes.data_as(C.POINTER(C.c_int32)),
        C.byref(calib) if calib is not None else None, C.byref(c), C.byref(g), C.byref(t)))
    return c.value, g.value, t.value


def _buf_array(shape, bufs: Sequence):
    arr = (C.c_void_p * shape.R)()
    for s in range(shape.R):
        b = bufs[s] if s < len(bufs) else None
        arr[s] = None if b is None else b.data_ptr()
    return arr


def moe_expert_forward_overlap(ctx: Context, shape, x_perm, w1, w3, w2, ws, h, y_perm, combine_bufs,
                               flags, epoch: int, n_consumer_cu: int, mode: int, stream=None):
    check("moe_expert_forward_overlap", lib().moe_expert_forward_overlap(
        ctx.handle, C.byref(shape), _ptr(x_perm), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws), _ptr(h),
        _ptr(y_perm), _buf_array(shape, combine_bufs), _ptr(flags), C.c_uint32(epoch),
        int(n_consumer_cu), int(mode), _stream(stream)))


def moe_expert_forward_gathered(ctx: Context, shape, x, w1, w3, w2, ws, h, y_perm, combine_bufs,
                                flags, epoch: int, n_consumer_cu: int, mode: int, stream=None):
    check("moe_expert_forward_gathered", lib().moe_expert_forward_gathered(
        ctx.handle, C.byref(shape), _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws), _ptr(h),
        _ptr(y_perm), _buf_array(shape, combine_bufs), _ptr(flags), C.c_uint32(epoch),
        int(n_consumer_cu), int(mode), _stream(stream)))


def moe_expert_forward_noalloc(ctx: Context, shape, x_perm, w1, w3, w2, ws, h, y_perm, combine_bufs,
                               flags, epoch: int, n_consumer_cu: int, mode: int, stream=None):
    check("moe_expert_forward_noalloc", lib().moe_expert_forward_noalloc(
        ctx.handle, C.byref(shape), _ptr(x_perm), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws), _ptr(h),
        _ptr(y_perm), _buf_array(shape, combine_bufs), _ptr(flags), C.c_uint32(epoch),
        int(n_consumer_cu), int(mode), _stream(stream)))


def moe_combine(shape, combine_bufs, y_perm, gates, ws, y_share, stream=None):
    check("moe_combine", lib().moe_combine(C.byref(shape), _buf_array(shape, combine_bufs),
                                           _ptr(y_perm), _ptr(gates), _ptr(ws), _ptr(y_share),
                                           _stream(stream)))


def moe_read_status(shape, ws, stream=None) -> int:
    st = C.c_int32()
    rc = lib().moe_read_status(C.byref(shape), _ptr(ws), C.byref(st), _stream(stream))
    if rc == _abi.MOE_ERR_HIP:
        raise _abi.MoeError("moe_read_status", rc)
    return st.value
