"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Each case monkeypatches one plausible bug into oracle.moe_share and checks
that at least one of the pin tests raises.
"""
import numpy as np
import pytest

from oracle import moe_share as om
import test_oracle_route_layout as RL
import test_oracle_ffn_combine as FC


def _route_ties_high(logits, k, gate_kind):
    lg = np.asarray(logits, dtype=np.float32)
    E = lg.shape[1]
    order = E - 1 - np.argsort(-lg[:, ::-1], axis=1, kind="stable")   # ties -> higher id
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    return ids, z / z.sum(axis=1, keepdims=True)


def _route_unnormalised(logits, k, gate_kind):
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)


def _silu_wrong_sign(u):
    return u / (1.0 + np.exp(u))


def _ffn_swapped(X, W1, W3, W2):
    if W3 is None:
        return om.silu(X @ W1.T) @ W2.T
    return (om.silu(X @ W3.T) * (X @ W1.T)) @ W2.T


def _order_local_first(R, r_self):
    return [r_self] + [s for s in range(R) if s != r_self]


MUTATIONS = {
    "ties_to_higher_id": ("route", _route_ties_high, [RL.test_route_ties_go_to_lower_expert_id]),
    "gates_not_renormalised": ("route", _route_unnormalised,
                               [lambda: RL.test_softmax_gates_equal_renormalised_full_softmax()]),
    "silu_sign": ("silu", _silu_wrong_sign,
                  [lambda: FC.test_sum_of_shares_equals_moe_definition(FC.TINY[0], 4)]),
    "w1_w3_swapped": ("expert_ffn", _ffn_swapped,
                      [lambda: FC.test_sum_of_shares_equals_moe_definition(FC.TINY[0], 1)]),
    "local_group_first": ("group_order", _order_local_first,
                          [lambda: RL.test_layout_matches_brute_force(4, 16, 8, 2, 0, 4)]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad, pins = MUTATIONS[name]
    monkeypatch.setattr(om, attr, bad)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


def test_dropped_gate_is_caught(monkeypatch):
    orig = om.weighted_reduction

    def no_gate(bufs, y_perm, gates, lay):
        return orig(bufs, y_perm, np.ones_like(gates), lay)
    monkeypatch.setattr(om, "weighted_reduction", no_gate)
    with pytest.raises(AssertionError):
        FC.test_sum_of_shares_equals_moe_definition(FC.TINY[1], 4)


def test_ascending_expert_order_is_caught(monkeypatch):
    def tile_schedule_ascending(lay):
        b = om.Bands.__new__(om.Bands)
        res = ORIG_SCHED(lay)
        # plant: reverse the order of experts' remote blocks
        n = res.n_remote
        blocks = []
        i = 0
        while i < n:
            j = i
            while j < n and res.expert[j] == res.expert[i]:
                j += 1
            blocks.append(list(range(i, j)))
            i = j
        perm = [p for blk in reversed(blocks) for p in blk] + list(range(n, len(res.row0)))
        for f in ("expert", "row0", "dest", "recv0", "valid"):
            setattr(b, f, getattr(res, f)[perm])
        b.n_remote = n
        return b
    monkeypatch.setattr(om, "tile_schedule", tile_schedule_ascending)
    with pytest.raises(AssertionError):
        RL.test_schedule_matches_page_example()


ORIG_SCHED = om.tile_schedule


# ------------------------------------------------ source-level planted mistakes

import inspect
import textwrap

from oracle import partition as op
import test_partition_model as PM


def _mutated(func, old, new):
    """A copy of func with one source fragment replaced (compiled in func's
    own module namespace, so it sees the same helpers)."""
    src = textwrap.dedent(inspect.getsource(func))
    assert old in src, f"mutation anchor not found in {func.__name__}: {old!r}"
    ns = dict(func.__globals__)
    exec(compile(src.replace(old, new, 1), f"<mutated {func.__name__}>", "exec"), ns)
    return ns[func.__name__]


def test_ties_by_expert_id_is_caught(monkeypatch):
    """Rule (ii) with the remote-rows key dropped (ties by expert id)."""
    bad = _mutated(om.tile_schedule, "key=lambda e: (-int(n_rb[e]), -int(n_rr[e]), e)",
                   "key=lambda e: (-int(n_rb[e]), e)")
    monkeypatch.setattr(om, "tile_schedule", bad)
    with pytest.raises(AssertionError):
        RL.test_schedule_equal_band_counts_more_remote_rows_first()


PARTITION_MUTATIONS = {
    # a row tile ready at the wave of its first instance, not its last
    "ready_at_first_instance": ("ready[p] = t_prod", "ready[p] = ready[p] or t_prod",
                                [PM.test_last_instance_sets_readiness]),
    # a partial wave priced at its full length
    "partial_wave_full_length": ("length * max(len(wave) / P, 1.0 / 3.0)", "length",
                                 [PM.test_single_tile_single_segment_closed_form,
                                  PM.test_whole_waves_of_identical_tiles]),
    # a segment's copy not queued behind the previous one
    "copies_in_parallel": ("t_copy = max(t_copy, start) +", "t_copy = start +",
                           [PM.test_segmented_group_closed_form]),
    # the copy moves only H bytes per row (a dropped factor 2 of bf16)
    "copy_bytes_halved": ("2.0 * H * int(segs.rows[i]) / bw", "H * int(segs.rows[i]) / bw",
                          [PM.test_single_tile_single_segment_closed_form]),
}


@pytest.mark.parametrize("name", sorted(PARTITION_MUTATIONS))
def test_partition_planted_mistake_is_caught(name, monkeypatch):
    old, new, pins = PARTITION_MUTATIONS[name]
    monkeypatch.setattr(op, "expert_phase_time", _mutated(op.expert_phase_time, old, new))
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
