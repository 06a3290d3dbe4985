"""Pins for the oracle's expert FFN, combine transfer and weighted reduction.

The reference values here come from the plain MoE definition evaluated token
by token with torch's CPU float64 ops (torch.nn.functional.silu, matmul), not
from the oracle's own layout/permute machinery.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from oracle import moe_share as om
from synth import Workload, make_expert_weights, make_logits, make_x, f32_to_bf16_bits


def tw(bits):
    return torch.from_numpy(om.widen_bf16(bits))


def dense_ffn_torch(x, w1, w3, w2):
    u = x @ w1.T
    h = Fnn.silu(u) * (x @ w3.T) if w3 is not None else Fnn.silu(u)
    return h @ w2.T


def all_expert_weights(w):
    return [make_expert_weights(w, e) for e in range(w.E)]


def moe_by_definition(w, logits, x_bits, weights):
    """y[g] = sum_j gate_j * FFN_{id_j}(x_g), token by token (sec. 2.1)."""
    ids, gates = om.route(logits, w.k, w.gate_kind)
    X = tw(x_bits.reshape(w.R * w.T, w.H))
    out = torch.zeros((w.R * w.T, w.H), dtype=torch.float64)
    for g in range(w.R * w.T):
        for j in range(w.k):
            w1, w3, w2 = weights[int(ids[g, j])]
            y = dense_ffn_torch(X[g:g + 1], tw(w1), tw(w3) if w3 is not None else None, tw(w2))
            out[g] += float(gates[g, j]) * y[0]
    return out.numpy().reshape(w.R, w.T, w.H)


def shares(w, logits, x_bits, weights, tb_m, mgb=1):
    El = w.E_local
    out = []
    for r in range(w.R):
        loc = weights[r * El:(r + 1) * El]
        W1 = np.stack([a for a, _, _ in loc])
        W3 = np.stack([b for _, b, _ in loc]) if w.gated else None
        W2 = np.stack([c for _, _, c in loc])
        out.append(om.oracle_share(logits, x_bits, W1, W3, W2, R=w.R, T=w.T, E=w.E, k=w.k,
                                   gate_kind=w.gate_kind, r_self=r, tb_m=tb_m, mgb=mgb))
    return out


TINY = [
    Workload("a", 4, 12, 16, 24, 8, 2, True, "softmax"),
    Workload("b", 2, 10, 8, 16, 4, 3, False, "softmax"),
    Workload("c", 4, 8, 16, 8, 16, 4, True, "sigmoid"),
]


@pytest.mark.parametrize("w", TINY, ids=lambda w: w.name)
@pytest.mark.parametrize("tb_m", [1, 4])
def test_sum_of_shares_equals_moe_definition(w, tb_m):
    logits, x = make_logits(w), make_x(w)
    weights = all_expert_weights(w)
    want = moe_by_definition(w, logits, x, weights)
    got = sum(r.y_share for r in shares(w, logits, x, weights, tb_m))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_identical_experts_equal_gates_reduce_to_dense_ffn():
    # closed form: identical experts and gates 1/k make the layer one dense FFN
    w = Workload("d", 4, 16, 16, 32, 8, 2, True, "softmax")
    rng = np.random.default_rng(9)
    logits = np.zeros((w.R * w.T, w.E), dtype=np.float32)
    for g in range(w.R * w.T):
        logits[g, rng.permutation(w.E)[:w.k]] = 1.0
    x = make_x(w)
    one = make_expert_weights(w, 0)
    weights = [one] * w.E
    got = sum(r.y_share for r in shares(w, logits, x, weights, 4))
    X = tw(x.reshape(-1, w.H))
    want = dense_ffn_torch(X, tw(one[0]), tw(one[1]), tw(one[2])).numpy().reshape(w.R, w.T, w.H)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_tokens_without_local_expert_are_exactly_zero():
    w = TINY[0]
    logits, x = make_logits(w), make_x(w)
    weights = all_expert_weights(w)
    res = shares(w, logits, x, weights, 4)[1]
    El = w.E_local
    ids = res.ids.reshape(w.R, w.T, w.k)
    none = ~((ids >= El) & (ids < 2 * El)).any(axis=2)
    assert none.any()
    assert np.all(res.y_share[none] == 0.0)
    assert np.any(res.y_share[~none] != 0.0)


def test_padding_rows_give_zero_outputs_and_are_not_transferred():
    w = TINY[0]
    logits, x = make_logits(w), make_x(w)
    weights = all_expert_weights(w)
    res = shares(w, logits, x, weights, 4)[0]
    pad = res.layout.row_src < 0
    assert pad.any()
    assert np.all(res.x_perm[pad] == 0) and np.all(res.y_perm[pad] == 0)
    for s, buf in enumerate(res.bufs):
        if buf is not None:
            assert buf.shape[0] == res.layout.counts[:, s].sum()


def test_w2_scaling_is_linear():
    w = TINY[0]
    logits, x = make_logits(w), make_x(w)
    weights = all_expert_weights(w)
    base = shares(w, logits, x, weights, 4)[0].y_share
    doubled = [(a, b, f32_to_bf16_bits(om.widen_bf16(c).astype(np.float32) * 2)) for a, b, c in weights]
    assert np.array_equal(shares(w, logits, x, doubled, 4)[0].y_share, 2 * base)


def test_token_rows_matches_full_share():
    w = TINY[2]
    logits, x = make_logits(w), make_x(w)
    weights = all_expert_weights(w)
    res = shares(w, logits, x, weights, 4)[2]
    El = w.E_local
    loc = weights[2 * El:3 * El]
    W1 = np.stack([a for a, _, _ in loc]); W3 = np.stack([b for _, b, _ in loc]); W2 = np.stack([c for _, _, c in loc])
    toks = [0, 5, 17, 31]
    got = om.token_rows(res, W1, W3, W2, toks)
    assert np.allclose(got, res.y_share.reshape(-1, w.H)[toks], rtol=1e-12, atol=1e-14)
