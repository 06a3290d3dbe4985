"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (default band height, partition-model consumer CU count).

Integer work (ids, counts, layout, schedule, plan, segments, row maps) is
compared bit-exactly with the oracle in full; x_perm and the combine
buffers are checked bit-exactly (rows against the source tokens / against
y_perm), and the gathered forward (no x_perm) against the materialized one;
expert outputs and the share are compared on sampled rows/tokens
against the fp64 oracle (one expert's weights widened at a time).
"""
import numpy as np
import pytest

from oracle import moe_share as om
from synth import WORKLOADS, make_local_weights, make_logits, make_x
from synth.workloads import ShareInputs
from parity_util import (assert_plan_equal, bits, check_row_tiles, check_rows, make_gpu_share,
                         oracle_plan_arrays, say, widen)
from test_gpu_parity import check_auto_partition, check_fused_gather, check_role_switch

pytestmark = pytest.mark.gpu

# (workload id, layer, band height) -- band heights as in bench.py
FULL = [(2, 0, 64), (3, 0, 256), (4, 0, 32), (5, 0, 64), (5, 2, 128)]


@pytest.mark.parametrize("wid,layer,tb", FULL, ids=[f"cfg{a}_l{b}_tb{c}" for a, b, c in FULL])
def test_full_size_parity(wid, layer, tb):
    import torch
    from combine_overlap_amd import MOE_CONSUMER_AUTO, MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL
    w = WORKLOADS[wid]
    say(f"[fullsize] {w.name} layer {layer} tb_m={tb}: inputs")
    W1, W3, W2 = make_local_weights(w, 0)
    inp = ShareInputs(w, 0, make_logits(w, layer), make_x(w), W1, W3, W2)
    sh, _ = make_gpu_share(w, 0, tb, None, inp)
    b = sh.buf
    mgb = sh.shape.mgb
    ref = om.oracle_share(inp.logits, inp.x, W1, W3, W2, R=w.R, T=w.T, E=w.E, k=w.k,
                          gate_kind=w.gate_kind, r_self=0, tb_m=tb, mgb=mgb, with_ffn=False)
    say(f"[fullsize] {w.name}: route + permute")
    sh.route()
    torch.cuda.synchronize()
    assert np.array_equal(b.topk_ids.cpu().numpy(), ref.ids)
    assert np.array_equal(b.counts.cpu().numpy(), ref.layout.counts)
    assert np.allclose(b.gates.cpu().numpy().astype(np.float64), ref.gates, rtol=2e-6, atol=1e-7)
    c, mgb2, _ = sh.partition()
    assert mgb2 == mgb
    sh.permute()
    plan = sh.plan_arrays()
    assert plan["status"] == 0
    assert_plan_equal(plan, oracle_plan_arrays(ref))
    check_row_tiles(plan, ref, sh.sizes.tile_m)
    check_auto_partition(sh, w.name)
    assert sh.auto_consumer_cu()[0] == c
    m_pad = plan["m_pad"]
    rng = np.random.default_rng(wid * 10 + layer)
    rows = rng.choice(m_pad, size=min(m_pad, 512), replace=False)
    assert np.array_equal(widen(b.x_perm[torch.from_numpy(rows).to(sh.device)]), ref.x_perm[rows])

    say(f"[fullsize] {w.name}: overlap c={c}")
    for s in range(w.R):
        if b.combine[s] is not None:
            b.combine[s].fill_(float("nan"))
    sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=c)
    sh.combine()
    torch.cuda.synchronize()
    assert sh.status() == 0
    y_bits = bits(b.y_perm[:m_pad])
    share_bits = bits(b.y_share).copy()
    # combine buffers hold exact copies of the remote bands' valid rows
    bd = ref.bands
    for i in range(bd.n_remote):
        s, r0, rc, n = int(bd.dest[i]), int(bd.row0[i]), int(bd.recv0[i]), int(bd.valid[i])
        got = b.combine[s][rc:rc + n].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, y_bits[r0:r0 + n]), f"band {i}"
    # sampled expert-output rows vs the fp64 FFN
    valid = np.nonzero(ref.layout.row_src >= 0)[0]
    pick = rng.choice(valid, size=min(valid.size, 96), replace=False)
    y_ref = np.zeros((pick.size, w.H))
    for e in range(w.E_local):
        lo, hi = ref.layout.expert_base[e], ref.layout.expert_base[e] + ref.layout.M_e[e]
        sel = np.nonzero((pick >= lo) & (pick < hi))[0]
        if sel.size:
            y_ref[sel] = om.expert_ffn(ref.x_perm[pick[sel]], om.widen_bf16(W1[e]),
                                       om.widen_bf16(W3[e]) if W3 is not None else None,
                                       om.widen_bf16(W2[e]))
    y_gpu = y_bits[pick].astype(np.uint32) << 16
    check_rows(y_gpu.view(np.float32).astype(np.float64), y_ref, f"{w.name} y_perm sample",
               layer_output=False)
    # sampled tokens of the share: with 0, 1 and several local slots
    nloc = ((ref.ids >= 0) & (ref.ids < w.E_local)).sum(axis=1)
    toks = []
    for want in sorted(set(nloc.tolist())):
        cand = np.nonzero(nloc == want)[0]
        toks += rng.choice(cand, size=min(cand.size, 24), replace=False).tolist()
    t_ref = om.token_rows(ref, W1, W3, W2, toks)
    t_gpu = (share_bits.reshape(-1, w.H)[toks].astype(np.uint32) << 16).view(np.float32)
    check_rows(t_gpu.astype(np.float64), t_ref, f"{w.name} y_share sample")

    say(f"[fullsize] {w.name}: sequential baseline")
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=c)
    sh.combine()
    torch.cuda.synchronize()
    assert np.array_equal(bits(b.y_perm[:m_pad]), y_bits)
    assert np.array_equal(bits(b.y_share), share_bits)

    say(f"[fullsize] {w.name}: the plan's own consumer count (no host round trip)")
    for mode in (MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL):
        for s in range(w.R):
            if b.combine[s] is not None:
                b.combine[s].fill_(float("nan"))
        sh.expert_forward(mode, n_consumer_cu=MOE_CONSUMER_AUTO)
        sh.combine()
        torch.cuda.synchronize()
        assert sh.status() == 0
        assert np.array_equal(bits(b.y_perm[:m_pad]), y_bits), f"mode {mode}: AUTO y_perm differs"
        assert np.array_equal(bits(b.y_share), share_bits), f"mode {mode}: AUTO y_share differs"

    say(f"[fullsize] {w.name}: gather fused into the first projection")
    check_fused_gather(sh, ref, w, w.name, c, y_bits, share_bits)

    say(f"[fullsize] {w.name}: role switching")
    check_role_switch(sh, ref, w, 0, w.name)


# (tokens per rank, N, experts per rank, router) of the tile-signalling
# paper's Table 2: its largest, most skewed corner and a small balanced one
TABLE2_CASES = [(16384, 8192, 64, "stress_skew"), (8192, 4096, 4, "balanced")]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tpr,N,E_l,router", TABLE2_CASES,
                         ids=[f"{r}_tpr{t}_n{n}_e{e}" for t, n, e, r in TABLE2_CASES])
def test_table2_shape_parity(tpr, N, E_l, router):
    """Shapes of the tile-signalling paper's Table 2 (sec. 4.1.3): the expert
    GEMM K = 2048 -> N as a non-gated FFN with F = 2048 and H = N, E_l
    experts per rank over 4 ranks, top-2 softmax; stress_skew routing =
    logits + ln Zipf(1.2) over the expert id (the hottest experts local to
    the timed rank), balanced = unbiased logits (readings of router modes
    the pages name but do not define). The plan in full, the combine buffers
    against y_perm bit for bit, sampled expert rows and tokens against the
    fp64 oracle, and every form (overlap at the model's c, sequential, role
    switching, the fused gather) with the same bits."""
    import torch
    from synth import Workload
    from combine_overlap_amd import MOE_CONSUMER_AUTO, MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL
    if router == "stress_skew":
        w = Workload(f"table2_stress_tpr{tpr}_n{N}_e{E_l}", 4, tpr, N, 2048, 4 * E_l, 2, False, "softmax",
                     "zipf", zipf_s=1.2, w_std="0.02")
    else:
        w = Workload(f"table2_balanced_tpr{tpr}_n{N}_e{E_l}", 4, tpr, N, 2048, 4 * E_l, 2, False, "softmax",
                     "normal", w_std="0.02")
    tb = 64
    say(f"[fullsize] {w.name}: inputs")
    W1, W3, W2 = make_local_weights(w, 0)
    inp = ShareInputs(w, 0, make_logits(w, 0), make_x(w), W1, W3, W2)
    sh, _ = make_gpu_share(w, 0, tb, None, inp)
    b = sh.buf
    ref = om.oracle_share(inp.logits, inp.x, W1, W3, W2, R=w.R, T=w.T, E=w.E, k=w.k, gate_kind=w.gate_kind,
                          r_self=0, tb_m=tb, mgb=sh.shape.mgb, with_ffn=False, with_rows=False)
    say(f"[fullsize] {w.name}: route + permute")
    sh.route()
    torch.cuda.synchronize()
    assert np.array_equal(b.topk_ids.cpu().numpy(), ref.ids)
    assert np.array_equal(b.counts.cpu().numpy(), ref.layout.counts)
    sh.permute()
    plan = sh.plan_arrays()
    assert plan["status"] == 0
    assert_plan_equal(plan, oracle_plan_arrays(ref))
    check_row_tiles(plan, ref, sh.sizes.tile_m)
    check_auto_partition(sh, w.name)
    m_pad = plan["m_pad"]
    rng = np.random.default_rng(2048)
    x_flat = inp.x.reshape(-1, w.H)
    valid = np.nonzero(ref.layout.row_src >= 0)[0]
    rows = rng.choice(valid, size=256, replace=False)
    got = b.x_perm[torch.from_numpy(rows).to(sh.device)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, x_flat[ref.layout.row_src[rows]]), "x_perm rows"

    c = sh.auto_consumer_cu()[0]
    say(f"[fullsize] {w.name}: overlap c={c}")
    for q in range(w.R):
        if b.combine[q] is not None:
            b.combine[q].fill_(float("nan"))
    sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=MOE_CONSUMER_AUTO)
    sh.combine()
    torch.cuda.synchronize()
    assert sh.status() == 0
    y_bits = bits(b.y_perm[:m_pad])
    share_bits = bits(b.y_share).copy()
    bd = ref.bands
    for i in range(bd.n_remote):
        s, r0, rc, n = int(bd.dest[i]), int(bd.row0[i]), int(bd.recv0[i]), int(bd.valid[i])
        got = b.combine[s][rc:rc + n].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, y_bits[r0:r0 + n]), f"band {i}"
    pick = rng.choice(valid, size=64, replace=False)
    y_ref = np.zeros((pick.size, w.H))
    for e in range(w.E_local):
        lo, hi = ref.layout.expert_base[e], ref.layout.expert_base[e] + ref.layout.M_e[e]
        sel = np.nonzero((pick >= lo) & (pick < hi))[0]
        if sel.size:
            X = om.widen_bf16(x_flat[ref.layout.row_src[pick[sel]]])
            y_ref[sel] = om.expert_ffn(X, om.widen_bf16(W1[e]), None, om.widen_bf16(W2[e]))
    y_gpu = (y_bits[pick].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    check_rows(y_gpu, y_ref, f"{w.name} y_perm sample", layer_output=False)
    nloc = ((ref.ids >= 0) & (ref.ids < w.E_local)).sum(axis=1)
    toks = []
    for want in sorted(set(nloc.tolist())):
        cand = np.nonzero(nloc == want)[0]
        toks += rng.choice(cand, size=min(cand.size, 16), replace=False).tolist()
    t_ref = om.token_rows(ref, W1, W3, W2, toks, x_bits=inp.x)
    t_gpu = (share_bits.reshape(-1, w.H)[toks].astype(np.uint32) << 16).view(np.float32)
    check_rows(t_gpu.astype(np.float64), t_ref, f"{w.name} y_share sample")

    say(f"[fullsize] {w.name}: sequential baseline, fused gather, role switching")
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=MOE_CONSUMER_AUTO)
    sh.combine()
    torch.cuda.synchronize()
    assert np.array_equal(bits(b.y_perm[:m_pad]), y_bits)
    assert np.array_equal(bits(b.y_share), share_bits)
    b.x_perm = None   # frees the materialized rows before the gathered run
    torch.cuda.empty_cache()
    sh.fused_gather = True
    try:
        sh.permute()
        for q in range(w.R):
            if b.combine[q] is not None:
                b.combine[q].fill_(float("nan"))
        sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=c)
        sh.combine()
        torch.cuda.synchronize()
        assert sh.status() == 0
        assert np.array_equal(bits(b.y_perm[:m_pad]), y_bits), "gathered y_perm"
        assert np.array_equal(bits(b.y_share), share_bits), "gathered y_share"
        check_role_switch(sh, ref, w, 0, w.name)
    finally:
        sh.fused_gather = False
