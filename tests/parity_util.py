"""Helpers for GPU-vs-oracle parity tests (imported by the -m gpu tests only)."""
from __future__ import annotations

import sys

import numpy as np

from oracle import moe_share as om
from synth import Workload, make_share_inputs

# Tolerance for floating-point outputs (bf16 storage, fp32 accumulation):
# per-row relative distance ||y - y_ref|| / ||y_ref|| <= REL_TOL and the
# element-wise bound below for every output; for the layer output (y_share)
# also the mean absolute error against the bf16-rounded reference
# <= MEAN_ABS_TOL. Intermediates (per-expert rows, combine buffers) are not
# gate-weighted, so their magnitude and hence their bf16 rounding floor is
# larger; they are held to the relative bounds only.
REL_TOL = 2e-2
MEAN_ABS_TOL = 2e-3
# element-wise relative error, each element against max(|ref|, the reference
# row's RMS): the same 2e-2 bound. A bf16 emulation of the gated FFN at the
# workloads' widths (fp32 accumulation, h and y rounded) gives at most 1.1e-2
# over a million elements, so the bound leaves room for the tails of larger
# outputs while one fully wrong element (error ~ the row's scale) fails it.
ELEM_TOL = 2e-2


def stated_default_calib(n_cu: int):
    """The CU-split model's calibration the library uses when none is given,
    as stated in its header (3.5 TFLOP/s per producer CU, b = 20 GB/s,
    B = 800 GB/s, 30 us for the last batch, candidates 8, 16, ..., 48), for
    the oracle. Written out here, not read from the library."""
    from oracle import partition as op
    c_max = min(n_cu - 1, 48)
    c_min = 8 if c_max >= 8 else max(1, c_max)
    return op.Calib(3.5e12, 0.0, 20e9, 800e9, 30e-6, n_cu, c_min, c_max, 8)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def widen(t) -> np.ndarray:
    """bf16 torch tensor -> float64 numpy (exact)."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_rows(got: np.ndarray, ref: np.ndarray, what: str, layer_output: bool = True):
    """Per-row relative distance, element-wise relative error against a
    per-row RMS floor, and (layer output) mean abs error vs bf16(ref)."""
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    nr = np.linalg.norm(ref, axis=1)
    zero = nr == 0
    assert np.all(got[zero] == 0), f"{what}: rows with zero reference are not exactly zero"
    rel = np.linalg.norm(got - ref, axis=1)[~zero] / nr[~zero]
    mae = float(np.mean(np.abs(got - bf16_round(ref)))) if got.size else 0.0
    mx = float(rel.max()) if rel.size else 0.0
    # element-wise: |got - ref| / max(|ref|, RMS of the reference row), so one
    # wrong element of a wide row cannot hide in the row's L2 distance while
    # elements near zero are held to the row's scale
    el = 0.0
    if np.any(~zero):
        g, r = got[~zero], ref[~zero]
        rms = (nr[~zero] / np.sqrt(ref.shape[-1]))[:, None]
        el = float((np.abs(g - r) / np.maximum(np.abs(r), rms)).max())
    say(f"  {what}: max per-row rel {mx:.3e}, max element rel {el:.3e}, mean abs err {mae:.3e}")
    assert mx <= REL_TOL, f"{what}: max per-row relative distance {mx} > {REL_TOL}"
    assert el <= ELEM_TOL, f"{what}: max element-wise relative error {el} > {ELEM_TOL}"
    if layer_output:
        assert mae <= MEAN_ABS_TOL, f"{what}: mean abs err {mae} > {MEAN_ABS_TOL}"
    return mx, mae


def make_gpu_share(w: Workload, r_self: int, tb_m: int, mgb: int, inp=None, device="cuda:0"):
    import torch
    from combine_overlap_amd.share import MoEShare, bf16_tensor
    if inp is None:
        inp = make_share_inputs(w, r_self)
    sh = MoEShare(w.R, w.T, w.H, w.F, w.E, w.k, w.gated, w.gate_kind, r_self=r_self, tb_m=tb_m,
                  mgb=mgb, device=device)
    d = sh.device
    sh.allocate(torch.from_numpy(inp.logits).to(d), bf16_tensor(inp.x, d), bf16_tensor(inp.W1, d),
                bf16_tensor(inp.W3, d) if inp.W3 is not None else None, bf16_tensor(inp.W2, d))
    return sh, inp


def oracle_plan_arrays(res: om.ShareResult) -> dict:
    lay, b, sg = res.layout, res.bands, res.segs
    return dict(
        m_pad=lay.m_pad, n_bands=len(b.row0), n_remote=b.n_remote, n_seg=len(sg.band0),
        group_row=lay.group_row, expert_base=lay.expert_base, recv_off=lay.recv_off,
        band_row0=b.row0, band_expert=b.expert, band_dest=b.dest, band_recv0=b.recv0,
        band_valid=b.valid, seg_band0=sg.band0, seg_nbands=sg.nbands, seg_dest=sg.dest,
        seg_src_row=sg.src_row, seg_dst_row=sg.dst_row, seg_rows=sg.rows,
        row_src=lay.row_src, recv_row=lay.recv_row)


def assert_plan_equal(got: dict, want: dict):
    for key, v in want.items():
        g = got[key]
        if np.isscalar(v) or isinstance(v, int):
            assert int(g) == int(v), f"{key}: {g} != {v}"
        else:
            g = np.asarray(g).reshape(np.shape(v))
            assert np.array_equal(g, np.asarray(v)), f"plan field {key} differs"


def check_row_tiles(plan: dict, res: om.ShareResult, tile_m: int):
    """The GEMM's row tiles (an implementation choice, not part of the method):
    they cut every expert's tb_m-aligned rows into tile_m pieces in layout
    order; the schedule is a permutation that lists every tile holding a
    remote band first (experts in the band schedule's order), then the rest by
    expert; every segment's tile range covers exactly its bands' rows."""
    lay, bd, sg = res.layout, res.bands, res.segs
    tb = lay.tb_m
    row0, ex, rows = plan["tile_row0"], plan["tile_expert"], plan["tile_rows"]
    want = []
    for e in range(lay.E_l):
        base = int(lay.expert_base[e])
        alg = -(-int(lay.M_e[e]) // tb) * tb
        for j in range(-(-alg // tile_m)):
            want.append((base + j * tile_m, e, min(tile_m, alg - j * tile_m)))
    got = list(zip(row0.tolist(), ex.tolist(), rows.tolist()))
    assert got == want, "row tiles do not cut the experts' aligned rows"
    sched = plan["tile_sched"].tolist()
    assert sorted(sched) == list(range(len(want))), "tile schedule is not a permutation"
    nrt = plan["n_remote_tiles"]
    remote_rows = {e: int(lay.group_row[e, lay.r_self]) - int(lay.expert_base[e]) for e in range(lay.E_l)}
    for pos, t in enumerate(sched):
        r0, e, _ = want[t]
        holds_remote = r0 - int(lay.expert_base[e]) < remote_rows[e]
        assert holds_remote == (pos < nrt), f"tile {t} at schedule position {pos}"
    # remote phase follows the band schedule's expert order
    order = []
    for e in bd.expert[:bd.n_remote].tolist():
        if not order or order[-1] != e:
            order.append(e)
    assert [want[t][1] for t in sched[:nrt]] == sorted([want[t][1] for t in sched[:nrt]],
                                                       key=order.index)
    for i in range(len(sg.band0)):
        first = int(bd.row0[sg.band0[i]])
        last = int(bd.row0[sg.band0[i] + sg.nbands[i] - 1]) + tb - 1
        t0, t1 = int(plan["seg_tile0"][i]), int(plan["seg_tile1"][i])
        assert want[t0][0] <= first < want[t0][0] + want[t0][2], f"segment {i} first tile"
        assert want[t1][0] <= last < want[t1][0] + want[t1][2], f"segment {i} last tile"
