"""Plain CPU oracle of the per-layer producer/consumer CU split.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module. It shares no
code with the HIP path: the row layout, band schedule and segments it works
on come from the oracle's own moe_share functions, and every step below is
an explicit event loop, not the library's closed form.

Sources:
  [Weave] abstract of "Weave: Fine-Grained Dynamic SM Scheduling in an MoE
    Megakernel for Compute-Communication Overlap" (arXiv 2609.21483): per
    layer and per GPU, from the routing result, the SMs are split into
    communication and computation workers so that the two groups'
    throughputs match the layer's communication/computation ratio.
  [TLS] "Fine-grained Computation-Communication Overlap via Tile-level
    Signaling and Scheduling for Mixture-of-Experts" (arXiv 2607.19539):
    sec. 4.3.4 / Fig. 9 (too few consumer SMs leave a long transfer tail, too
    many slow the GEMM); sec. 3.3.2 / Fig. 3(a) (transfer bandwidth saturates
    only at MiB-scale writes); sec. 3.2.2 (the remote-first schedule whose
    tiles the producer runs).

Reading (the pages give no formula; this is the plainest model that uses
only the routing counts and measured rates). For c consumer CUs out of n_cu:
  * the producer runs the output projection on P = n_cu - c CUs. Its work is
    the GEMM row tiles (tile_m rows of one expert's tb_m-aligned rows, the
    last one shorter) in the GEMM schedule order: every row tile holding a
    remote band first, experts in the band schedule's order, then the others
    by expert id. Each row tile has ceil(H / tile_n) column-tile instances;
    one instance takes 2 * rows32 * tile_n * F / rate(M_e) seconds on one CU
    (rows32 = the tile's rows rounded up to 32, the MFMA block height;
    rate(M) = gemm_flops_per_cu * M / (M + gemm_m_half), M_e the expert's
    packed rows);
  * the instances run in order, in waves of P: a wave lasts as long as its
    slowest instance; a partial last wave of n < P instances lasts that
    times max(n / P, 1/3) (fewer tiles share the memory system);
  * a row tile is ready when the wave holding its last instance ends;
  * the consumer copies the segments in schedule order; a segment starts
    once all row tiles holding its bands are ready and the previous copy has
    ended, and moves 2 H bytes per valid row at BW(c) = c b / (1 + c b / B)
    (b = copy_bw_per_cu, B = copy_bw_max);
  * the layer's expert phase takes T(c) = max(producer end, copy end +
    seg_latency_s), or the producer end when nothing is copied;
  * c is the candidate with the least T(c) (the smallest c on equal times);
  * segment size: mgb = 2 when one band moves less than half a MiB, else 1.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import moe_share as om


@dataclasses.dataclass
class Calib:
    """Rates of the model (measured on the device) and the candidate range."""

    gemm_flops_per_cu: float   # FLOP/s of one producer CU on the output projection
    gemm_m_half: float         # rows per expert at which the rate halves (0: constant)
    copy_bw_per_cu: float      # b, bytes/s one consumer CU moves beside the GEMM
    copy_bw_max: float         # B, bytes/s the copy saturates at
    seg_latency_s: float       # fixed cost of the copy's last batch
    n_cu: int
    c_min: int
    c_max: int
    c_step: int

    def candidates(self) -> List[int]:
        return list(range(self.c_min, self.c_max + 1, self.c_step))


def segment_bands(tb_m: int, H: int) -> int:
    """Bands per middle segment: 2 when one band (tb_m rows of 2 H bytes)
    is under half a MiB, else 1 ([TLS] Fig. 3(a): small writes run far below
    the bandwidth plateau)."""
    return 2 if 2 * tb_m * H < 0.5 * 1048576 else 1


@dataclasses.dataclass
class RowTile:
    expert: int
    row0: int        # first packed row
    rows: int        # rows of the expert's tb_m-aligned rows it holds
    remote: bool     # holds a remote band


def gemm_row_tiles(lay: om.Layout, bands: om.Bands, tile_m: int) -> List[RowTile]:
    """The producer's row tiles in its schedule order (remote-holding tiles
    first, experts in the band schedule's order; then the rest by expert id)."""
    tiles: Dict[int, List[RowTile]] = {}
    for e in range(lay.E_l):
        base = int(lay.expert_base[e])
        aligned = -(-int(lay.M_e[e]) // lay.tb_m) * lay.tb_m
        remote_rows = int(lay.group_row[e, lay.r_self]) - base   # the local group is last
        tiles[e] = [RowTile(e, base + j * tile_m, min(tile_m, aligned - j * tile_m), j * tile_m < remote_rows)
                    for j in range(-(-aligned // tile_m))]
    order: List[int] = []
    for e in bands.expert[:bands.n_remote].tolist():
        if e not in order:
            order.append(int(e))
    sched = [t for e in order for t in tiles[e] if t.remote]
    sched += [t for e in range(lay.E_l) for t in tiles[e] if not t.remote]
    return sched


def expert_phase_time(sched: List[RowTile], segs: om.Segments, bands: om.Bands, lay: om.Layout, *,
                      H: int, F: int, c: int, calib: Calib, tile_n: int = 256) -> float:
    """T(c) of the model for one candidate, simulated event by event."""
    P = calib.n_cu - c
    per_tile = -(-H // tile_n)

    def tile_time(t: RowTile) -> float:
        m = max(int(lay.M_e[t.expert]), 1)
        rate = calib.gemm_flops_per_cu * m / (m + calib.gemm_m_half)
        rows32 = -(-t.rows // 32) * 32
        return 2.0 * rows32 * tile_n * F / rate

    instances = [p for p in range(len(sched)) for _ in range(per_tile)]
    ready = [0.0] * len(sched)
    t_prod = 0.0
    for w0 in range(0, len(instances), P):
        wave = instances[w0:w0 + P]
        length = max(tile_time(sched[p]) for p in wave)
        t_prod += length if len(wave) == P else length * max(len(wave) / P, 1.0 / 3.0)
        for p in wave:
            ready[p] = t_prod          # later waves overwrite: the last instance's wave
    if len(segs.band0) == 0:
        return t_prod
    # the row tile holding each packed row (a band never straddles two row
    # tiles: tb_m divides tile_m and both start at the expert's base)
    pos_of_row = {}
    for p, t in enumerate(sched):
        for r in range(t.row0, t.row0 + t.rows):
            pos_of_row[r] = p
    bw = c * calib.copy_bw_per_cu / (1.0 + c * calib.copy_bw_per_cu / calib.copy_bw_max)
    t_copy = 0.0
    for i in range(len(segs.band0)):
        b0 = int(segs.band0[i])
        start = max(ready[pos_of_row[int(bands.row0[b])]] for b in range(b0, b0 + int(segs.nbands[i])))
        t_copy = max(t_copy, start) + 2.0 * H * int(segs.rows[i]) / bw
    return max(t_prod, t_copy + calib.seg_latency_s)


@dataclasses.dataclass
class Partition:
    c: int
    mgb: int
    predicted_s: float
    times: Dict[int, float]


def partition_model(counts: np.ndarray, *, R: int, H: int, F: int, tb_m: int, r_self: int, calib: Calib,
                    mgb: Optional[int] = None, tile_m: int = 256, tile_n: int = 256) -> Partition:
    """Consumer CU count for one layer from its routing counts [E_l, R].

    mgb None takes the model's own segment size (segment_bands); a given mgb
    evaluates the model on that segmentation (the layout's plan as built)."""
    counts = np.asarray(counts, dtype=np.int64)
    E_l = counts.shape[0]
    lay = om.counts_layout(counts, R, 1, E_l, r_self, tb_m)
    bands = om.tile_schedule(lay)
    g = segment_bands(tb_m, H) if mgb is None else int(mgb)
    segs = om.segments(bands, g)
    sched = gemm_row_tiles(lay, bands, tile_m)
    times = {c: expert_phase_time(sched, segs, bands, lay, H=H, F=F, c=c, calib=calib, tile_n=tile_n)
             for c in calib.candidates()}
    best = min(times, key=lambda c: (times[c], c))
    return Partition(best, g, times[best], times)
