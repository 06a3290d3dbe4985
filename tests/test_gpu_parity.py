"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work (routing ids, counts, layout, schedule, plan, segments, row
maps) and byte copies (x_perm, combine buffers) must match bit-exactly;
floating-point outputs must satisfy the per-row relative distance and mean
absolute error bounds of parity_util.
"""
import numpy as np
import pytest

from oracle import moe_share as om
from synth import Workload, WORKLOADS, make_share_inputs
from parity_util import (assert_plan_equal, bits, check_row_tiles, check_rows, make_gpu_share,
                         oracle_plan_arrays, say, stated_default_calib, widen)

pytestmark = pytest.mark.gpu

# (id, workload, r_self, tb_m, mgb, consumer CUs, layer)
CASES = [
    ("tiny_full_tb64", WORKLOADS[1], 0, 64, 1, 4, 0),
    ("tiny_full_tb128_r2", WORKLOADS[1], 2, 128, 2, 2, 0),
    # more consumer workgroups than copy units: one unit per workgroup, the
    # rest copy nothing and join the producer at once
    ("tiny_full_c48", WORKLOADS[1], 0, 64, 2, 48, 0),
    ("mixtral_mini_tb128", Workload("mixtral_mini", 4, 512, 1024, 2048, 8, 2, True, "softmax",
                                    "normal", w_std="fan_in"), 0, 128, 1, 8, 0),
    ("zipf_mini_tb256", Workload("zipf_mini", 4, 512, 1024, 1024, 8, 2, True, "softmax", "zipf",
                                 w_std="fan_in"), 0, 256, 2, 8, 0),
    ("fine_mini_tb64", Workload("fine_mini", 8, 256, 512, 256, 64, 8, True, "sigmoid"), 3, 64, 1, 16, 0),
    ("dyn_mini_tb64_l2", Workload("dyn_mini", 4, 512, 512, 384, 32, 8, True, "softmax", "layered",
                                  layers=16), 0, 64, 2, 6, 2),
    ("ragged_T300_R3", Workload("ragged", 3, 300, 256, 128, 6, 3, True, "softmax"), 1, 64, 1, 3, 0),
    ("single_rank", Workload("single", 1, 100, 256, 256, 4, 2, False, "softmax"), 0, 64, 1, 2, 0),
    ("k_equals_E", Workload("kE", 2, 64, 256, 128, 4, 4, True, "sigmoid"), 1, 128, 1, 2, 0),
    # bands of 32 rows under 256-row GEMM tiles: tiles span several owners' bands
    ("fine_mini_tb32", Workload("fine_mini", 8, 256, 512, 256, 64, 8, True, "sigmoid"), 0, 32, 2, 8, 0),
    ("zipf_mini_tb32", Workload("zipf_mini", 4, 512, 1024, 1024, 8, 2, True, "softmax", "zipf",
                                w_std="fan_in"), 2, 32, 3, 8, 0),
    # 16-row bands: an expert's last 32-row MFMA block may hold the next expert's rows
    ("fine_mini_tb16", Workload("fine_mini", 8, 256, 512, 256, 64, 8, True, "sigmoid"), 1, 16, 2, 8, 0),
    ("ragged_tb16", Workload("ragged", 3, 300, 256, 128, 6, 3, True, "softmax"), 2, 16, 1, 3, 0),
    # degenerate and limit cases: no row for this rank at all (empty layout,
    # no tiles, no segments); the most source ranks (16) with k = 16; the most
    # experts (512, 256 of them local); one token per rank
    ("no_local_rows", Workload("nolocal", 4, 128, 256, 128, 8, 2, True, "softmax"), 1, 64, 1, 8, 0,
     "no_local"),
    ("max_ranks_k16", Workload("maxfan", 16, 64, 256, 128, 64, 16, True, "sigmoid"), 5, 16, 2, 8, 0),
    ("max_experts", Workload("maxE", 2, 128, 256, 128, 512, 8, True, "softmax"), 1, 32, 1, 8, 0),
    ("one_token_per_rank", Workload("one", 4, 1, 256, 128, 8, 2, True, "softmax"), 3, 64, 1, 2, 0),
    # non-gated FFN with F % 256 != 0: the first projection runs 256 x 128 tiles
    ("nongated_f384", Workload("ng384", 4, 256, 512, 384, 8, 2, False, "softmax"), 2, 64, 1, 4, 0),
    # 16 experts: routing with one lane per token and 16 logits per lane
    ("experts16_k4", Workload("e16", 4, 200, 256, 256, 16, 4, True, "softmax"), 1, 32, 1, 4, 0),
    # top-1 routing; H = 768 (three output column tiles, a combine row of 96
    # 16-byte steps) and gated F = 384 (three first-projection column tiles)
    ("top1_h768_f384", Workload("top1", 4, 256, 768, 384, 8, 1, True, "softmax"), 2, 64, 1, 4, 0),
]


def _inputs(w, r_self, layer, modifier=None):
    from synth import make_logits, make_x, make_local_weights
    from synth.workloads import ShareInputs
    W1, W3, W2 = make_local_weights(w, r_self)
    logits = make_logits(w, layer)
    if modifier == "no_local":
        # this rank's experts are never among any token's top k
        El = w.E // w.R
        logits = logits.copy()
        logits[:, r_self * El:(r_self + 1) * El] = -30.0
    return ShareInputs(w, r_self, logits, make_x(w), W1, W3, W2)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_share_parity(case):
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL
    name, w, r_self, tb, mgb, c, layer = case[:7]
    modifier = case[7] if len(case) > 7 else None
    say(f"[parity] {name}: R={w.R} T={w.T} H={w.H} F={w.F} E={w.E} k={w.k} r_self={r_self} "
        f"tb_m={tb} mgb={mgb} c={c}")
    inp = _inputs(w, r_self, layer, modifier)
    ref = om.oracle_share(inp.logits, inp.x, inp.W1, inp.W3, inp.W2, R=w.R, T=w.T, E=w.E, k=w.k,
                          gate_kind=w.gate_kind, r_self=r_self, tb_m=tb, mgb=mgb)
    sh, _ = make_gpu_share(w, r_self, tb, mgb, inp)
    b = sh.buf

    # step 1: routing
    sh.route()
    torch.cuda.synchronize()
    assert np.array_equal(b.topk_ids.cpu().numpy(), ref.ids), "topk ids differ"
    assert np.array_equal(b.counts.cpu().numpy(), ref.layout.counts), "counts differ"
    g = b.gates.cpu().numpy().astype(np.float64)
    assert np.allclose(g, ref.gates, rtol=2e-6, atol=1e-7), f"gates differ {np.abs(g - ref.gates).max()}"

    # steps 3-4: layout, schedule, plan, segments, gather
    sh.permute()
    plan = sh.plan_arrays()
    assert plan["status"] == 0
    assert_plan_equal(plan, oracle_plan_arrays(ref))
    check_row_tiles(plan, ref, sh.sizes.tile_m)
    m_pad = plan["m_pad"]
    assert np.array_equal(widen(b.x_perm[:m_pad]), ref.x_perm), "x_perm differs"
    check_auto_partition(sh, name)

    # expert FFN + overlapped transfer
    for s in range(w.R):
        if b.combine[s] is not None:
            b.combine[s].fill_(float("nan"))
    b.y_perm.fill_(float("nan"))
    sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=c)
    torch.cuda.synchronize()
    assert sh.status() == 0
    y_gpu = widen(b.y_perm[:m_pad])
    check_rows(y_gpu, ref.y_perm, f"{name} y_perm", layer_output=False)
    y_bits = bits(b.y_perm[:m_pad])
    comb = {s: bits(b.combine[s]) for s in range(w.R) if s != r_self}
    for i in range(len(ref.bands.row0)):
        if i >= ref.bands.n_remote:
            break
        s, r0, rc, n = (int(ref.bands.dest[i]), int(ref.bands.row0[i]), int(ref.bands.recv0[i]),
                        int(ref.bands.valid[i]))
        assert np.array_equal(comb[s][rc:rc + n], y_bits[r0:r0 + n]), f"combine buf band {i} differs"
    for s in comb:
        check_rows(widen(b.combine[s][:int(ref.layout.recv_rows[s])]), ref.bufs[s], f"{name} combine[{s}]",
                   layer_output=False)

    # weighted reduction
    sh.combine()
    torch.cuda.synchronize()
    y_share_ovl = bits(b.y_share).copy()
    check_rows(widen(b.y_share), ref.y_share, f"{name} y_share")

    # the non-overlapped baseline with the same consumer count gives bit-identical results
    for s in range(w.R):
        if b.combine[s] is not None:
            b.combine[s].fill_(float("nan"))
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=c)
    sh.combine()
    torch.cuda.synchronize()
    assert np.array_equal(bits(b.y_perm[:m_pad]), y_bits), "sequential y_perm differs from overlap"
    assert np.array_equal(bits(b.y_share), y_share_ovl), "sequential y_share differs from overlap"

    # the gather fused into the first projection: same bits as the materialized path
    check_fused_gather(sh, ref, w, name, c, y_bits, y_share_ovl)

    # role switching: the producer's workgroups copy; same bits as SEQUENTIAL with c = 0
    check_role_switch(sh, ref, w, r_self, name)


def check_auto_partition(sh, name):
    """The plan kernel's evaluation of the CU-split model (MOE_CONSUMER_AUTO)
    against the oracle's event simulation of the model on the same counts and
    segment size, with the library's stated default calibration: the same c
    (an argmin of the oracle's times) and the predicted time to 1e-9. The
    host function moe_plan_partition against the oracle with the model's own
    segment size."""
    from oracle import partition as op
    c_dev, t_dev = sh.auto_consumer_cu()
    counts = sh.buf.counts.cpu().numpy()
    shp = sh.shape
    cal = stated_default_calib(sh.ctx.num_cus)
    kw = dict(R=shp.R, H=shp.H, F=shp.F, tb_m=shp.tb_m, r_self=shp.r_self, calib=cal)
    ref = op.partition_model(counts, mgb=shp.mgb, **kw)
    say(f"  {name}: CU split device c={c_dev} ({t_dev:.9e} s), oracle c={ref.c} ({ref.predicted_s:.9e} s)")
    assert t_dev != -1.0, f"{name}: the plan's model tables overflowed"
    assert c_dev in ref.times, f"{name}: device c {c_dev} is not a candidate"
    best = min(ref.times.values())
    assert ref.times[c_dev] == pytest.approx(best, rel=1e-9), f"{name}: device c {c_dev} is not the argmin"
    runner_up = min([t for c, t in ref.times.items() if c != ref.c], default=float("inf"))
    if runner_up > best * (1 + 1e-9):
        assert c_dev == ref.c, f"{name}: device c {c_dev} != oracle c {ref.c}"
    assert t_dev == pytest.approx(ref.predicted_s, rel=1e-9), f"{name}: predicted {t_dev!r} != {ref.predicted_s!r}"
    c_host, g_host, t_host = sh.partition()
    ref_h = op.partition_model(counts, **kw)
    assert g_host == ref_h.mgb
    assert ref_h.times[c_host] == pytest.approx(min(ref_h.times.values()), rel=1e-9)
    assert t_host == pytest.approx(ref_h.predicted_s, rel=1e-9)


def check_fused_gather(sh, ref, w, name, c, y_bits, share_bits):
    """moe_permute without x_perm builds the same plan and indexes (row_src is
    -1 on every padding row whatever the workspace held before), and
    moe_expert_forward_gathered, whose first projection reads the rows straight
    from x, gives the bits of the materialized overlapped run with the same c:
    y_perm (padding rows included), the combine buffers and the share."""
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, ops
    b = sh.buf
    m_pad = int(ref.layout.m_pad)
    # stale indexes that a missing padding pass would leave: every row -> token 0
    v = ops.moe_plan_view(sh.shape, b.ws)
    o = (v["row_src"] - b.ws.data_ptr()) // 4
    b.ws.view(torch.int32)[o:o + int(sh.sizes.m_pad_max)].fill_(0)
    sh.fused_gather = True
    try:
        sh.permute()
        plan = sh.plan_arrays()
        assert plan["status"] == 0
        assert_plan_equal(plan, oracle_plan_arrays(ref))
        for s in range(w.R):
            if b.combine[s] is not None:
                b.combine[s].fill_(float("nan"))
        b.h.fill_(float("nan"))
        b.y_perm.fill_(float("nan"))
        sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=c)
        sh.combine()
        torch.cuda.synchronize()
        assert sh.status() == 0
        got = bits(b.y_perm[:m_pad])
        assert np.array_equal(got, y_bits), f"{name}: gathered y_perm differs from the materialized run"
        bd = ref.bands
        for i in range(bd.n_remote):
            s, r0, rc, n = int(bd.dest[i]), int(bd.row0[i]), int(bd.recv0[i]), int(bd.valid[i])
            assert np.array_equal(bits(b.combine[s][rc:rc + n]), got[r0:r0 + n]), f"{name}: gathered band {i}"
        assert np.array_equal(bits(b.y_share), share_bits), f"{name}: gathered y_share differs"
    finally:
        sh.fused_gather = False


def check_role_switch(sh, ref, w, r_self, name):
    import torch
    from combine_overlap_amd import MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL
    b = sh.buf
    m_pad = int(ref.layout.m_pad)
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=0)
    sh.combine()
    torch.cuda.synchronize()
    seq_y, seq_share = bits(b.y_perm[:m_pad]).copy(), bits(b.y_share).copy()
    for s in range(w.R):
        if b.combine[s] is not None:
            b.combine[s].fill_(float("nan"))
    sh.expert_forward(MOE_MODE_ROLE_SWITCH)
    sh.combine()
    torch.cuda.synchronize()
    assert sh.status() == 0
    y_bits = bits(b.y_perm[:m_pad])
    assert np.array_equal(y_bits, seq_y), f"{name}: role-switch y_perm differs from sequential"
    bd = ref.bands
    for i in range(bd.n_remote):
        s, r0, rc, n = int(bd.dest[i]), int(bd.row0[i]), int(bd.recv0[i]), int(bd.valid[i])
        assert np.array_equal(bits(b.combine[s][rc:rc + n]), y_bits[r0:r0 + n]), f"{name}: role-switch band {i}"
    assert np.array_equal(bits(b.y_share), seq_share), f"{name}: role-switch y_share differs from sequential"


def test_repeated_overlap_calls_are_deterministic():
    """Repeated calls with one consumer count give identical bits; every
    consumer count (which also sizes the output projection's K-split tail)
    stays within tolerance of the oracle."""
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL
    w = Workload("rep", 4, 512, 1024, 1024, 8, 2, True, "softmax", "zipf", w_std="fan_in")
    say("[parity] repeated overlap calls, epochs 1..12, c in 1,2,4,8,16,32")
    sh, inp = make_gpu_share(w, 0, 128, 1)
    ref = om.oracle_share(inp.logits, inp.x, inp.W1, inp.W3, inp.W2, R=w.R, T=w.T, E=w.E, k=w.k,
                          gate_kind=w.gate_kind, r_self=0, tb_m=128, mgb=1)
    sh.route()
    sh.permute()
    for c in (1, 2, 4, 8, 16, 32):
        outs = []
        for mode in (MOE_MODE_OVERLAP, MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL):
            for s in range(w.R):
                if sh.buf.combine[s] is not None:
                    sh.buf.combine[s].fill_(float("nan"))
            sh.expert_forward(mode, n_consumer_cu=c)
            sh.combine()
            torch.cuda.synchronize()
            assert sh.status() == 0
            outs.append(bits(sh.buf.y_share).copy())
        assert np.array_equal(outs[1], outs[0]), f"c={c}: repeated overlap calls differ"
        assert np.array_equal(outs[2], outs[0]), f"c={c}: sequential differs from overlap"
        check_rows(widen(sh.buf.y_share), ref.y_share, f"rep c={c} y_share")
