"""The per-layer CU-split model: the oracle pinned, the library against it.

The oracle (oracle.partition) simulates the model's definition event by
event. Its pins are special cases whose value follows by hand from the
definition (a single tile and segment; producer-only layers; a row tile whose
instances span two waves; exact multiples of the producer count), bounds
any schedule must respect, and monotonicity in the rates. The host library's
moe_plan_partition evaluates the same model in a closed form; it must agree
with the oracle on every candidate c to rounding and pick the oracle's c.
"""
import numpy as np
import pytest

from combine_overlap_amd import _abi, ops
from oracle import partition as op
from parity_util import stated_default_calib

# a calibration with round numbers for the hand-derived cases
SIMPLE = dict(gemm_flops_per_cu=1e12, gemm_m_half=0.0, copy_bw_per_cu=10e9, copy_bw_max=1e12,
              seg_latency_s=1e-6)


def calib(n_cu, c_min, c_max, c_step, **kw):
    d = dict(SIMPLE)
    d.update(kw)
    return op.Calib(n_cu=n_cu, c_min=c_min, c_max=c_max, c_step=c_step, **d)


def bw(cal, c):
    return c * cal.copy_bw_per_cu / (1 + c * cal.copy_bw_per_cu / cal.copy_bw_max)


# ---------------------------------------------------------------- oracle pins

def test_single_tile_single_segment_closed_form():
    # one expert, 40 rows from the one remote rank, band 64: one row tile of
    # 64 rows, one column tile (H = 256), one segment of 40 valid rows. One
    # instance on P >= 208 CUs is a partial wave: t_tile / 3. The copy starts
    # then and moves 2 H 40 bytes. T(c) = t_tile / 3 + 2 H 40 / BW(c) + L.
    cal = calib(256, 8, 48, 8)
    H, F = 256, 1024
    t_tile = 2.0 * 64 * 256 * F / cal.gemm_flops_per_cu
    res = op.partition_model(np.array([[0, 40]]), R=2, H=H, F=F, tb_m=64, r_self=0, calib=cal)
    for c, t in res.times.items():
        want = t_tile / 3 + 2.0 * H * 40 / bw(cal, c) + cal.seg_latency_s
        assert t == pytest.approx(want, rel=1e-12), c
    assert res.c == 48           # the copy is all that varies: the widest consumer wins
    assert res.mgb == 2          # a 64 x 256 band is 32 KiB, under half a MiB


def test_segmented_group_closed_form():
    # 300 remote rows in bands of 64: 5 bands (320 rows), two row tiles of
    # 256 and 64 rows, both in one partial wave ending at t_256 / 3. Segments
    # 1, 2, 1, 1 bands carry 64, 128, 64 and 44 valid rows; all start at the
    # same ready time, so the copy ends at t_256 / 3 + 2 H 300 / BW(c).
    cal = calib(256, 8, 48, 8)
    H, F = 256, 1024
    t256 = 2.0 * 256 * 256 * F / cal.gemm_flops_per_cu
    res = op.partition_model(np.array([[0, 300]]), R=2, H=H, F=F, tb_m=64, r_self=0, calib=cal)
    for c, t in res.times.items():
        assert t == pytest.approx(t256 / 3 + 2.0 * H * 300 / bw(cal, c) + cal.seg_latency_s, rel=1e-12)


def test_last_instance_sets_readiness():
    # P = 8 producer CUs (n_cu 10, c 2); two row tiles of 256 remote rows
    # (band = tile = 256) with 5 column tiles each (H = 1280): wave 0 holds
    # instances 0..7 (all of tile 0, three of tile 1), the partial wave 1 the
    # last two of tile 1 (length t / 3). Tile 0 is ready at t, tile 1 at 4t/3.
    # One band moves 640 KiB (>= half a MiB): segments of one band each.
    cal = calib(10, 2, 2, 1)
    H, F = 1280, 4096
    t = 2.0 * 256 * 256 * F / cal.gemm_flops_per_cu
    cp = 2.0 * H * 256 / bw(cal, 2)
    end0 = t + cp
    end1 = max(end0, 4 * t / 3) + cp
    want = max(4 * t / 3, end1 + cal.seg_latency_s)
    res = op.partition_model(np.array([[0, 512]]), R=2, H=H, F=F, tb_m=256, r_self=0, calib=cal)
    assert res.mgb == 1
    assert res.times[2] == pytest.approx(want, rel=1e-12)


def test_whole_waves_of_identical_tiles():
    # no remote rows: 2048 local rows = 8 row tiles of 256, 3 column tiles
    # each (H = 768): 24 instances. With P = 8 (c = 2 of 10) they fill exactly
    # 3 waves: T = 3 t. With P = 6 (c = 4): 4 waves, T = 4 t. With P = 5
    # (c = 5): 4 whole waves and a partial one of 4 instances: T = 4 t + t 4/5.
    cal = calib(10, 2, 5, 1)
    H, F = 768, 2048
    t = 2.0 * 256 * 256 * F / cal.gemm_flops_per_cu
    res = op.partition_model(np.array([[2048, 0]]), R=2, H=H, F=F, tb_m=64, r_self=0, calib=cal)
    assert res.times[2] == pytest.approx(3 * t, rel=1e-12)
    assert res.times[4] == pytest.approx(4 * t, rel=1e-12)
    assert res.times[5] == pytest.approx(4 * t + t * 4 / 5, rel=1e-12)
    assert res.c == 2


def test_no_copy_small_layer_ties_to_smallest_c():
    # 100 local rows: one short tile (128 rows computed as 4 x 32) and one
    # instance: every candidate gives t / 3, the smallest c wins the tie
    cal = calib(256, 8, 48, 8)
    res = op.partition_model(np.array([[100, 0, 0, 0]]), R=4, H=256, F=512, tb_m=32, r_self=0, calib=cal)
    t = 2.0 * 128 * 256 * 512 / cal.gemm_flops_per_cu
    assert all(v == pytest.approx(t / 3, rel=1e-12) for v in res.times.values())
    assert res.c == 8


def test_short_tile_rows_round_to_mfma_blocks():
    # 33 local rows: the tile computes 64 rows (two 32-row blocks)
    cal = calib(256, 8, 8, 8)
    res = op.partition_model(np.array([[33, 0]]), R=2, H=256, F=512, tb_m=16, r_self=0, calib=cal)
    assert res.times[8] == pytest.approx(2.0 * 64 * 256 * 512 / cal.gemm_flops_per_cu / 3, rel=1e-12)


def _random_counts(rng, El, R, kind, tb):
    if kind == "uniform":
        return rng.integers(0, 4 * tb + 7, size=(El, R))
    if kind == "skew":
        return (rng.pareto(1.2, size=(El, R)) * 300).astype(np.int64)
    return rng.integers(0, 3, size=(El, R)) * rng.integers(0, 2000, size=(El, R))


@pytest.mark.parametrize("seed", range(6))
def test_bounds_and_monotonicity(seed):
    rng = np.random.default_rng(seed)
    R, El, H, F, tb = 4, 6, 1024, 1536, 64
    counts = _random_counts(rng, El, R, ("uniform", "skew", "sparse")[seed % 3], tb)
    cal = calib(64, 2, 16, 2)
    res = op.partition_model(counts, R=R, H=H, F=F, tb_m=tb, r_self=1, calib=cal)
    remote = int(counts.sum() - counts[:, 1].sum())
    lay = op.om.counts_layout(counts, R, 1, El, 1, tb)
    work = sum(2.0 * (-(-t.rows // 32) * 32) * 256 * F / cal.gemm_flops_per_cu * (H // 256)
               for t in op.gemm_row_tiles(lay, op.om.tile_schedule(lay), 256))
    for c, t in res.times.items():
        assert t >= work / (cal.n_cu - c) * (1 - 1e-12)                         # producer work bound
        if remote:
            assert t >= 2.0 * H * remote / bw(cal, c) + cal.seg_latency_s - 1e-15  # copy bound
    faster_copy = calib(64, 2, 16, 2, copy_bw_per_cu=20e9, copy_bw_max=2e12)
    faster_gemm = calib(64, 2, 16, 2, gemm_flops_per_cu=2e12)
    for other in (faster_copy, faster_gemm):
        r2 = op.partition_model(counts, R=R, H=H, F=F, tb_m=tb, r_self=1, calib=other)
        for c in res.times:
            assert r2.times[c] <= res.times[c] * (1 + 1e-12)
    assert res.times[res.c] == min(res.times.values())


# ------------------------------------------------- library closed form vs oracle

CASES = [
    # R, E, H, F, k, tb, r_self, counts generator
    (4, 8, 4096, 14336, 2, 64, 0, "uniform"),
    (8, 256, 7168, 2048, 8, 32, 0, "uniform"),
    (4, 128, 4096, 1536, 8, 64, 1, "skew"),
    (4, 16, 8192, 2048, 2, 128, 0, "skew"),
    (2, 4, 2048, 1024, 2, 256, 1, "sparse"),
    (3, 6, 1024, 512, 3, 32, 2, "uniform"),
]


def _lib_calib(cal):
    return _abi.MoeCalib(cal.gemm_flops_per_cu, cal.gemm_m_half, cal.copy_bw_per_cu, cal.copy_bw_max,
                         cal.seg_latency_s, cal.n_cu, cal.c_min, cal.c_max, cal.c_step)


@pytest.mark.parametrize("case", CASES, ids=[f"R{c[0]}_E{c[1]}_tb{c[5]}_{c[7]}" for c in CASES])
@pytest.mark.parametrize("which", ["mi355x_like", "halfrate"])
def test_library_matches_oracle(case, which):
    R, E, H, F, k, tb, r_self, kind = case
    El = E // R
    rng = np.random.default_rng(R * 1000 + E + tb)
    counts = _random_counts(rng, El, R, kind, tb).astype(np.int32)
    if which == "mi355x_like":
        cal = op.Calib(3.5e12, 0.0, 20e9, 800e9, 30e-6, 256, 8, 48, 8)
    else:
        cal = op.Calib(2e12, 512.0, 35e9, 2e12, 5e-6, 128, 2, 20, 2)
    sh = ops.make_shape(R, 1 << 14, H, F, E, k, r_self, True, "softmax", tb, 1)
    ref = op.partition_model(counts, R=R, H=H, F=F, tb_m=tb, r_self=r_self, calib=cal)
    c_lib, g_lib, t_lib = ops.moe_plan_partition(sh, counts, _lib_calib(cal))
    assert g_lib == ref.mgb
    assert c_lib == ref.c
    assert t_lib == pytest.approx(ref.predicted_s, rel=1e-9)
    # every candidate: the library's prediction for a one-value range
    for c, t in ref.times.items():
        one = _abi.MoeCalib(cal.gemm_flops_per_cu, cal.gemm_m_half, cal.copy_bw_per_cu, cal.copy_bw_max,
                            cal.seg_latency_s, cal.n_cu, c, c, 1)
        assert ops.moe_plan_partition(sh, counts, one)[2] == pytest.approx(t, rel=1e-9), f"c={c}"


def test_library_default_calibration_matches_stated_values():
    """The library's built-in calibration (calib = NULL) is the one the GPU
    tests hand the oracle: 3.5 TFLOP/s per producer CU, b = 20 GB/s,
    B = 800 GB/s, 30 us, candidates 8, 16, ..., 48 of 256 CUs."""
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 3000, size=(2, 4)).astype(np.int32)
    sh = ops.make_shape(4, 4096, 4096, 14336, 8, 2, 0, True, "softmax", 64, 1)
    c_lib, g_lib, t_lib = ops.moe_plan_partition(sh, counts)
    ref = op.partition_model(counts, R=4, H=4096, F=14336, tb_m=64, r_self=0, calib=stated_default_calib(256))
    assert (c_lib, g_lib) == (ref.c, ref.mgb)
    assert t_lib == pytest.approx(ref.predicted_s, rel=1e-9)

