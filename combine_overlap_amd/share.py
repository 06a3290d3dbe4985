"""One EP rank's MoE-layer share on one GPU: buffer ownership + call order.

MoEShare allocates every device buffer the C ABI needs for one shape and runs
route -> permute -> (partition) -> expert forward (overlap or sequential) ->
combine, all through the HIP library. PyTorch only provides device memory,
streams and events. With fused_gather the routed rows are not copied into
x_perm: permute builds the indexes only and the expert forward's first
projection reads them from x (moe_expert_forward_gathered).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import _abi
from . import ops


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bf16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


@dataclasses.dataclass
class ShareBuffers:
    logits: torch.Tensor
    x: torch.Tensor
    w1: torch.Tensor
    w3: Optional[torch.Tensor]
    w2: torch.Tensor
    topk_ids: torch.Tensor
    gates: torch.Tensor
    counts: torch.Tensor
    ws: torch.Tensor
    x_perm: Optional[torch.Tensor]   # None while the gather is fused
    h: torch.Tensor
    y_perm: torch.Tensor
    combine: list
    flags: torch.Tensor
    y_share: torch.Tensor


class MoEShare:
    """Buffers and launch sequence for rank r_self's share of one MoE layer."""

    def __init__(self, R, T, H, F, E, k, gated, gate_kind, r_self=0, tb_m=128, mgb=None,
                 device="cuda:0", fused_gather=False):
        self.device = torch.device(device)
        self.fused_gather = bool(fused_gather)
        self.shape = ops.make_shape(R, T, H, F, E, k, r_self, gated, gate_kind, tb_m, mgb or 1)
        self.sizes = ops.moe_query_sizes(self.shape)
        self.R, self.T, self.H, self.F, self.E, self.k = R, T, H, F, E, k
        self.El = E // R
        self.r_self = r_self
        self.gated = bool(gated)
        self.ctx = ops.Context()
        self.epoch = 0
        self.buf: Optional[ShareBuffers] = None
        self.counts_host = torch.empty((self.El, R), dtype=torch.int32, pin_memory=True)
        self.counts_ready = torch.cuda.Event()
        # the segment size depends on the shape only; the CU split needs the counts
        self.shape.mgb = ops.moe_plan_partition(self.shape, np.zeros((self.El, R), np.int32))[1] \
            if mgb is None else mgb

    # ------------------------------------------------------------ buffers
    def allocate(self, logits: torch.Tensor, x: torch.Tensor, w1, w3, w2) -> ShareBuffers:
        d, s = self.device, self.sizes
        R, T, H, F, k, El = self.R, self.T, self.H, self.F, self.k, self.El
        mp = int(s.m_pad_max)
        ws = torch.empty(int(s.ws_bytes) + 256, dtype=torch.uint8, device=d)
        off = (-ws.data_ptr()) % 256
        ws = ws[off:off + int(s.ws_bytes)]
        combine = [None if q == self.r_self else
                   torch.empty((max(1, s.recv_rows_max), H), dtype=torch.bfloat16, device=d)
                   for q in range(R)]
        self.buf = ShareBuffers(
            logits=logits, x=x, w1=w1, w3=w3, w2=w2,
            topk_ids=torch.empty((R * T, k), dtype=torch.int32, device=d),
            gates=torch.empty((R * T, k), dtype=torch.float32, device=d),
            counts=torch.empty((El, R), dtype=torch.int32, device=d),
            ws=ws,
            x_perm=None if self.fused_gather else torch.empty((mp, H), dtype=torch.bfloat16, device=d),
            h=torch.empty((mp, F), dtype=torch.bfloat16, device=d),
            y_perm=torch.empty((mp, H), dtype=torch.bfloat16, device=d),
            combine=combine,
            flags=torch.zeros(max(1, s.max_flags), dtype=torch.int32, device=d),
            y_share=torch.empty((R, T, H), dtype=torch.bfloat16, device=d),
        )
        return self.buf

    def set_routing(self, tb_m: Optional[int] = None, mgb: Optional[int] = None):
        """Changes the band height / segment size (the buffers were sized for the
        tb_m given at construction: only equal or smaller tb_m fit)."""
        sh = self.shape
        if tb_m is not None:
            new = ops.make_shape(sh.R, sh.T, sh.H, sh.F, sh.E, sh.k, sh.r_self, sh.gated,
                                 sh.gate_kind, tb_m, sh.mgb)
            if ops.moe_query_sizes(new).ws_bytes > self.sizes.ws_bytes:
                raise ValueError("buffers too small for this tb_m")
            sh.tb_m = tb_m
        if mgb is not None:
            sh.mgb = mgb

    # ------------------------------------------------------------ steps
    def route(self, stream=None):
        b = self.buf
        ops.moe_route(self.shape, b.logits, b.topk_ids, b.gates, b.counts, b.ws, stream)

    def permute(self, stream=None):
        b = self.buf
        if self.fused_gather:
            ops.moe_permute(self.shape, None, b.topk_ids, b.counts, None, b.ws, stream)
            return
        if b.x_perm is None:
            b.x_perm = torch.empty((int(self.sizes.m_pad_max), self.H), dtype=torch.bfloat16,
                                   device=self.device)
        ops.moe_permute(self.shape, b.x, b.topk_ids, b.counts, b.x_perm, b.ws, stream)

    def partition(self, calib=None):
        cnt = self.buf.counts.cpu().numpy()
        return ops.moe_plan_partition(self.shape, cnt, calib)

    def expert_forward(self, mode=_abi.MOE_MODE_OVERLAP, n_consumer_cu=8, stream=None):
        b = self.buf
        self.epoch = (self.epoch % 0xFFFFFFF0) + 1
        fwd = ops.moe_expert_forward_gathered if self.fused_gather else ops.moe_expert_forward_overlap
        fwd(self.ctx, self.shape, b.x if self.fused_gather else b.x_perm, b.w1, b.w3, b.w2, b.ws, b.h,
            b.y_perm, b.combine, b.flags, self.epoch, n_consumer_cu, mode, stream)

    def combine(self, stream=None):
        b = self.buf
        ops.moe_combine(self.shape, b.combine, b.y_perm, b.gates, b.ws, b.y_share, stream)

    def forward(self, mode=_abi.MOE_MODE_OVERLAP, n_consumer_cu=8, stream=None):
        self.route(stream)
        self.permute(stream)
        self.expert_forward(mode, n_consumer_cu, stream)
        self.combine(stream)

    def layer(self, mode=_abi.MOE_MODE_OVERLAP, n_consumer_cu: Optional[int] = None, calib=None,
              stream=None) -> int:
        """The whole share with the per-layer CU split: route, permute, expert
        phase, combine. By default the plan kernel picks the consumer CU count
        on the device (MOE_CONSUMER_AUTO) and the host never waits. With a
        calibration the host evaluates the partition model instead: the counts
        go to pinned host memory (async) and the permute runs while the host
        waits for them. Returns the consumer CU count passed to the forward."""
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        self.route(s)
        if n_consumer_cu is None and calib is not None:
            with torch.cuda.stream(s):
                self.counts_host.copy_(self.buf.counts, non_blocking=True)
            self.counts_ready.record(s)
            self.permute(s)
            self.counts_ready.synchronize()
            n_consumer_cu = ops.moe_plan_partition(self.shape, self.counts_host.numpy(), calib)[0]
        else:
            self.permute(s)
            if n_consumer_cu is None:
                n_consumer_cu = _abi.MOE_CONSUMER_AUTO
        self.expert_forward(mode, n_consumer_cu, s)
        self.combine(s)
        return n_consumer_cu

    def auto_consumer_cu(self):
        """(consumer CUs, predicted seconds) the last permute's plan chose on the device."""
        torch.cuda.synchronize(self.device)
        v = ops.moe_plan_view(self.shape, self.buf.ws)
        o = (v["meta"] - self.buf.ws.data_ptr()) // 4
        meta = self.buf.ws.view(torch.int32)[o:o + _abi.META_PRED + 2].cpu().numpy()
        return int(meta[_abi.META_CAUTO]), float(meta[_abi.META_PRED:].view(np.float64)[0])

    def status(self, stream=None) -> int:
        return ops.moe_read_status(self.shape, self.buf.ws, stream)

    # ------------------------------------------------------------ inspection
    def plan_arrays(self) -> dict:
        """Copies the plan arrays of the workspace to host numpy arrays."""
        torch.cuda.synchronize(self.device)
        v = ops.moe_plan_view(self.shape, self.buf.ws)
        base = self.buf.ws.data_ptr()
        ws_i32 = self.buf.ws.view(torch.int32)

        def arr(name, n):
            o = (v[name] - base) // 4
            return ws_i32[o:o + n].cpu().numpy().copy()
        meta = arr("meta", 8)
        m_pad, n_bands, n_remote, n_seg = (int(meta[i]) for i in range(4))
        El, R = self.El, self.R
        out = dict(meta=meta, m_pad=m_pad, n_bands=n_bands, n_remote=n_remote, n_seg=n_seg,
                   status=int(meta[_abi.META_STATUS]))
        out["group_row"] = arr("group_row", El * R).reshape(El, R)
        out["expert_base"] = arr("expert_base", El + 1)
        out["recv_off"] = arr("recv_off", R * El).reshape(R, El)
        for f in ("band_row0", "band_expert", "band_dest", "band_recv0", "band_valid"):
            out[f] = arr(f, n_bands)
        for f in ("seg_band0", "seg_nbands", "seg_dest", "seg_src_row", "seg_dst_row", "seg_rows"):
            out[f] = arr(f, n_seg)
        n_tiles = int(meta[_abi.META_NTILES])
        out["n_tiles"] = n_tiles
        out["n_remote_tiles"] = int(meta[_abi.META_NRTILES])
        for f in ("tile_row0", "tile_expert", "tile_rows", "tile_sched"):
            out[f] = arr(f, n_tiles)
        for f in ("seg_tile0", "seg_tile1"):
            out[f] = arr(f, n_seg)
        out["row_src"] = arr("row_src", m_pad)
        out["recv_row"] = arr("recv_row", self.R * self.T * self.k).reshape(self.R * self.T, self.k)
        return out
