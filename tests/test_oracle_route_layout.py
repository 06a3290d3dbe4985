"""Pins for the oracle's routing, row layout, schedule and segments.

Each check is independent of the oracle's own code: brute-force enumeration
on tiny inputs, library special cases (scipy softmax / expit), the page's
worked scheduling example, and invariants the pages state in prose.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe_share as om
from synth import Workload, make_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_ids(rng, R, T, E, k):
    """Random distinct top-k ids per token (a routing, not a router output)."""
    return np.array([rng.permutation(E)[:k] for _ in range(R * T)], dtype=np.int32)


# ---------------------------------------------------------------- routing

def brute_topk(logits, k):
    out = []
    for row in logits:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (64, 8), (5, 5)])
def test_route_ids_match_full_sort(E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = rng.standard_normal((200, E)).astype(np.float32)
    ids, _ = om.route(logits, k, "softmax")
    assert np.array_equal(ids, brute_topk(logits, k))


def test_route_ties_go_to_lower_expert_id():
    logits = np.array([[1, 3, 3, 0, 3, 2]], dtype=np.float32)
    ids, _ = om.route(logits, 4, "softmax")
    assert ids.tolist() == [[1, 2, 4, 5]]
    logits = np.zeros((3, 8), dtype=np.float32)
    ids, g = om.route(logits, 3, "softmax")
    assert ids.tolist() == [[0, 1, 2]] * 3
    assert np.allclose(g, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_route_selected_dominate_unselected():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((500, 32)).astype(np.float32)
    ids, _ = om.route(logits, 6, "sigmoid")
    for i in range(logits.shape[0]):
        sel = set(ids[i].tolist())
        assert len(sel) == 6
        lo = min(logits[i, list(sel)])
        hi = max(logits[i, [e for e in range(32) if e not in sel]])
        assert lo >= hi


def test_softmax_gates_equal_renormalised_full_softmax():
    # special case reducing to a library routine: softmax over the selected k
    # equals the full softmax restricted to the selected experts and renormalised
    rng = np.random.default_rng(4)
    logits = (3 * rng.standard_normal((300, 16))).astype(np.float32)
    ids, g = om.route(logits, 4, "softmax")
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    ps = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(g, ps / ps.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    assert np.all(np.diff(g, axis=1) <= 0)          # highest logit -> largest gate
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_softmax_top2_closed_form():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    ids, g = om.route(logits, 2, "softmax")
    l = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    assert np.allclose(g[:, 0], scipy.special.expit(l[:, 0] - l[:, 1]), rtol=1e-13, atol=0)


def test_sigmoid_gates_normalised():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((300, 256)).astype(np.float32)
    ids, g = om.route(logits, 8, "sigmoid")
    sg = scipy.special.expit(np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1))
    assert np.allclose(g, sg / sg.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


# ---------------------------------------------------------------- layout

def brute_layout_rows(ids, R, T, E_l, r_self, tb_m, e):
    """Expected rows of X_e, by direct enumeration of the rules of sec. 3.2.1."""
    glob = r_self * E_l + e
    rows = []
    for s in [r for r in range(R) if r != r_self] + [r_self]:
        grp = [s * T + t for t in range(T) if glob in ids[s * T + t].tolist()]
        rows += grp
        if s != r_self:
            rows += [-1] * ((-len(grp)) % tb_m)
    return rows


LAYOUT_CASES = [
    # R, T, E, k, r_self, tb_m
    (4, 16, 8, 2, 0, 4), (4, 16, 8, 2, 2, 4), (3, 10, 6, 3, 1, 2),
    (2, 12, 4, 4, 1, 1), (4, 9, 8, 8, 3, 4), (2, 7, 2, 1, 0, 4), (1, 8, 4, 2, 0, 4),
]


@pytest.mark.parametrize("R,T,E,k,r_self,tb_m", LAYOUT_CASES)
def test_layout_matches_brute_force(R, T, E, k, r_self, tb_m):
    rng = np.random.default_rng(R * 1000 + T * 10 + tb_m)
    ids = tiny_ids(rng, R, T, E, k)
    E_l = E // R
    lay = om.row_layout(ids, R, T, E_l, r_self, tb_m)
    base = 0
    for e in range(E_l):
        want = brute_layout_rows(ids, R, T, E_l, r_self, tb_m, e)
        assert lay.expert_base[e] == base
        assert lay.M_e[e] == len(want)
        got = lay.row_src[base:base + len(want)].tolist()
        assert got == want
        nxt = base + (-(-len(want) // tb_m)) * tb_m
        assert all(v == -1 for v in lay.row_src[base + len(want):nxt])
        base = nxt
    assert lay.m_pad == base


@pytest.mark.parametrize("R,T,E,k,r_self,tb_m", LAYOUT_CASES)
def test_layout_invariants(R, T, E, k, r_self, tb_m):
    rng = np.random.default_rng(R * 7 + T + tb_m)
    ids = tiny_ids(rng, R, T, E, k)
    E_l = E // R
    lay = om.row_layout(ids, R, T, E_l, r_self, tb_m)
    first = r_self * E_l
    # each token appears once per local slot
    n_local = ((ids >= first) & (ids < first + E_l)).sum(axis=1)
    occ = np.bincount(lay.row_src[lay.row_src >= 0], minlength=R * T)
    assert np.array_equal(occ, n_local)
    # every token of every rank is routed k times over all E experts
    assert np.all(np.bincount(ids.ravel(), minlength=E).sum() == R * T * k)
    # padding only on remote owner boundaries, at most tb_m-1 rows per group,
    # so at most (R-1)(tb_m-1) per expert (sec. 4.5, read per expert)
    pad = lay.padded - lay.counts
    assert np.all(pad[:, r_self] == 0)
    assert np.all(pad <= tb_m - 1)
    assert np.all(pad.sum(axis=1) <= (R - 1) * (tb_m - 1))
    # groups start tile-aligned inside X_e
    for e in range(E_l):
        for s in range(R):
            assert (lay.group_row[e, s] - lay.expert_base[e]) % tb_m == 0
    # receive offsets tile [0, rows for s) without overlap, expert by expert
    for s in range(R):
        ends = lay.recv_off[s] + lay.counts[:, s]
        assert lay.recv_off[s, 0] == 0
        assert np.array_equal(lay.recv_off[s, 1:], ends[:-1])
        assert ends[-1] == lay.recv_rows[s]


def test_layout_tb1_is_plain_counting_sort():
    rng = np.random.default_rng(11)
    R, T, E, k = 4, 20, 8, 3
    ids = tiny_ids(rng, R, T, E, k)
    lay = om.row_layout(ids, R, T, 2, 1, 1)
    assert lay.m_pad == lay.counts.sum()
    hist = lay.counts[:, [0, 2, 3, 1]].reshape(-1)       # group order 0,2,3 then self
    offs = np.concatenate([[0], np.cumsum(hist)[:-1]])
    assert np.array_equal(lay.group_row[:, [0, 2, 3, 1]].reshape(-1), offs)


def test_recv_row_points_back_to_token():
    rng = np.random.default_rng(12)
    R, T, E, k, r_self, tb = 4, 24, 8, 3, 2, 4
    ids = tiny_ids(rng, R, T, E, k)
    lay = om.row_layout(ids, R, T, 2, r_self, tb)
    b = om.tile_schedule(lay)
    # invert the plan: receive-buffer row -> packed row, from the bands alone
    recv_to_row = {}
    for i in range(b.n_remote):
        for q in range(b.valid[i]):
            recv_to_row[(int(b.dest[i]), int(b.recv0[i]) + q)] = int(b.row0[i]) + q
    first = r_self * 2
    for g in range(R * T):
        s = g // T
        for j in range(k):
            r = lay.recv_row[g, j]
            if not (first <= ids[g, j] < first + 2):
                assert r == -1
                continue
            row = r if s == r_self else recv_to_row[(s, int(r))]
            assert lay.row_src[row] == g
            e = ids[g, j] - first
            assert lay.expert_base[e] <= row < lay.expert_base[e] + lay.M_e[e]


# ---------------------------------------------------------------- schedule

def test_schedule_matches_page_example():
    with open(os.path.join(GOLDEN, "fig2c_rank1_schedule.json")) as f:
        fx = json.load(f)
    R, T, E, r_self, tb = fx["R"], fx["T"], fx["E"], fx["r_self"], fx["tb_m"]
    ids = np.array(fx["ids"], dtype=np.int32)
    E_l = E // R
    lay = om.row_layout(ids, R, T, E_l, r_self, tb)
    b = om.tile_schedule(lay)
    first = r_self * E_l
    remote_experts = [k for k, _ in itertools.groupby((b.expert[:b.n_remote] + first).tolist())]
    assert remote_experts == fx["expected_remote_expert_order_global"]
    assert np.all(b.dest[:b.n_remote] != r_self)
    assert np.all(b.dest[b.n_remote:] == r_self)
    local_experts = [k for k, _ in itertools.groupby((b.expert[b.n_remote:] + first).tolist())]
    assert local_experts == fx["expected_local_expert_order_global"]


@pytest.mark.parametrize("R,T,E,k,r_self,tb_m", LAYOUT_CASES)
def test_schedule_invariants(R, T, E, k, r_self, tb_m):
    rng = np.random.default_rng(R + T + E + k + tb_m)
    ids = tiny_ids(rng, R, T, E, k)
    E_l = E // R
    lay = om.row_layout(ids, R, T, E_l, r_self, tb_m)
    b = om.tile_schedule(lay)
    nb = len(b.row0)
    # rule (i): remote bands first
    assert np.all(b.dest[:b.n_remote] != r_self) and np.all(b.dest[b.n_remote:] == r_self)
    # each expert's remote bands are contiguous, experts in non-increasing band count
    seq = [k for k, _ in itertools.groupby(b.expert[:b.n_remote].tolist())]
    assert len(seq) == len(set(seq))
    cnt = [int(np.sum(b.expert[:b.n_remote] == e)) for e in seq]
    assert cnt == sorted(cnt, reverse=True)
    # bands cover every row of every X_e at band granularity, once
    covered = np.zeros(lay.m_pad, dtype=int)
    for i in range(nb):
        covered[b.row0[i]:b.row0[i] + tb_m] += 1
        rows = lay.row_src[b.row0[i]:b.row0[i] + tb_m]
        owners = {int(g) // T for g in rows if g >= 0}
        assert owners == {int(b.dest[i])}                 # single destination per tile
        assert b.valid[i] == int(np.sum(rows >= 0))       # padding never transferred
        assert np.all(rows[:b.valid[i]] >= 0)
    for e in range(E_l):
        lo = lay.expert_base[e]
        span = (-(-lay.M_e[e] // tb_m)) * tb_m
        assert np.all(covered[lo:lo + span] == 1)
    # receive placements of remote bands do not overlap and fill each buffer
    for s in range(R):
        if s == r_self:
            continue
        mark = np.zeros(lay.recv_rows[s], dtype=int)
        for i in range(b.n_remote):
            if b.dest[i] == s:
                mark[b.recv0[i]:b.recv0[i] + b.valid[i]] += 1
        assert np.all(mark == 1)


@pytest.mark.parametrize("mgb", [1, 2, 3])
def test_segments_partition_groups(mgb):
    rng = np.random.default_rng(40 + mgb)
    R, T, E, k, r_self, tb = 4, 64, 8, 2, 0, 2
    ids = tiny_ids(rng, R, T, E, k)
    lay = om.row_layout(ids, R, T, 2, r_self, tb)
    b = om.tile_schedule(lay)
    sg = om.segments(b, mgb)
    # consecutive, covering all remote bands exactly once
    assert sg.band0[0] == 0
    assert np.array_equal(sg.band0[1:], (sg.band0 + sg.nbands)[:-1])
    assert sg.band0[-1] + sg.nbands[-1] == b.n_remote
    # per (expert, dest) group: 1, x, ..., x, (rest), 1
    for key, grp in itertools.groupby(range(len(sg.band0)),
                                      key=lambda i: (int(b.expert[sg.band0[i]]), int(sg.dest[i]))):
        grp = list(grp)
        sizes = [int(sg.nbands[i]) for i in grp]
        if len(sizes) >= 2:
            assert sizes[0] == 1 and sizes[-1] == 1
            mid = sizes[1:-1]
            assert all(m == mgb for m in mid[:-1]) and all(1 <= m <= mgb for m in mid)
        for i in grp:
            p = sg.band0[i]
            assert np.all(b.expert[p:p + sg.nbands[i]] == key[0])
            assert np.all(b.dest[p:p + sg.nbands[i]] == key[1])
            assert sg.rows[i] == b.valid[p:p + sg.nbands[i]].sum()
            assert sg.src_row[i] == b.row0[p] and sg.dst_row[i] == b.recv0[p]


def test_page_padding_bound_per_expert_at_scale():
    # sec. 4.5: padding rows per owner boundary < tb_m, so (W-1)(tb_m-1) per expert
    w = Workload("t", 4, 2048, 8, 8, 64, 2, True, "softmax", "zipf")
    ids, _ = om.route(make_logits(w), 2, "softmax")
    for tb in (16, 64, 256):
        lay = om.row_layout(ids, 4, 2048, 16, 0, tb)
        pad = (lay.padded - lay.counts).sum(axis=1)
        assert np.all(pad <= 3 * (tb - 1))


def test_schedule_equal_band_counts_more_remote_rows_first():
    """[TLS] sec. 3.2.2 rule (ii) on a tie of Algorithm 1's band count: the
    expert with more remote rows goes first (tests/golden fixture)."""
    with open(os.path.join(GOLDEN, "rule2_equal_bands_more_rows_first.json")) as f:
        fx = json.load(f)
    R, T, E, r_self, tb = fx["R"], fx["T"], fx["E"], fx["r_self"], fx["tb_m"]
    ids = np.array(fx["ids"], dtype=np.int32)
    E_l = E // R
    lay = om.row_layout(ids, R, T, E_l, r_self, tb)
    b = om.tile_schedule(lay)
    first = r_self * E_l
    remote = b.expert[:b.n_remote] + first
    for e, n in fx["expected_remote_band_counts_by_expert"].items():
        assert int(np.sum(remote == int(e))) == n
        assert int(b.valid[:b.n_remote][remote == int(e)].sum()) == fx["expected_remote_rows_by_expert"][e]
    assert [k for k, _ in itertools.groupby(remote.tolist())] == fx["expected_remote_expert_order_global"]
    local = [k for k, _ in itertools.groupby((b.expert[b.n_remote:] + first).tolist())]
    assert local == fx["expected_local_expert_order_global"]
