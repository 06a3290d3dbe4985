"""The seeded input generators against the recipe they state.

They hold none of the method's arithmetic; these tests pin what every parity
test and the bench rely on: the bf16 rounding of the drawn values (checked
against torch's own fp32 -> bf16 conversion), reproducibility, the stated
value distributions and routing skews, and the weight scales.
"""
import numpy as np
import pytest

from synth import Workload, WORKLOADS, make_logits, make_x
from synth.workloads import (bf16_bits_to_f32, f32_to_bf16_bits, layer_temperatures, make_expert_weights,
                             zipf_probs)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000),
        # exact ties between two bf16 values (round half to even) and their neighbours
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38], dtype=np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(a), ref)
    # widening is exact: a bf16 value survives the round trip
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(ref)), ref)


def test_bf16_nan_stays_nan():
    b = f32_to_bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_f32(b)).all()


def test_generators_are_reproducible_and_keyed():
    w = Workload("repro", 2, 64, 256, 128, 8, 2, True, "softmax", "zipf")
    assert np.array_equal(make_logits(w), make_logits(w))
    assert np.array_equal(make_x(w), make_x(w))
    a, b, c = make_expert_weights(w, 3)
    a2, b2, c2 = make_expert_weights(w, 3)
    assert np.array_equal(a, a2) and np.array_equal(b, b2) and np.array_equal(c, c2)
    # a different expert, seed or tensor gives different values
    assert not np.array_equal(make_expert_weights(w, 4)[0], a)
    assert not np.array_equal(make_x(w.replace(seed=1)), make_x(w))
    assert not np.array_equal(a, b)


def test_activations_are_standard_normal():
    w = Workload("xdist", 2, 512, 1024, 128, 8, 2, True, "softmax")
    x = bf16_bits_to_f32(make_x(w)).astype(np.float64)
    assert x.shape == (2, 512, 1024)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert abs((np.abs(x) < 1.0).mean() - 0.6827) < 0.01


@pytest.mark.parametrize("wid", [2, 4])
def test_weight_scale_follows_the_stated_rule(wid):
    w = WORKLOADS[wid].replace(H=1024, F=512)   # same rule at a smaller size
    w1, w3, w2 = make_expert_weights(w, 0)
    s1 = bf16_bits_to_f32(w1).std()
    s2 = bf16_bits_to_f32(w2).std()
    if w.w_std == "fan_in":
        assert s1 == pytest.approx(1024 ** -0.5, rel=0.02)
        assert s2 == pytest.approx(512 ** -0.5, rel=0.02)
    else:
        assert s1 == pytest.approx(0.02, rel=0.02)
        assert s2 == pytest.approx(0.02, rel=0.02)
    assert w1.shape == (512, 1024) and w2.shape == (1024, 512)
    assert w3 is not None and w3.shape == w1.shape


def _top1_share(logits):
    E = logits.shape[1]
    return np.bincount(np.argmax(logits, axis=1), minlength=E) / logits.shape[0]


def test_normal_routing_is_balanced():
    w = Workload("bal", 4, 4096, 64, 64, 8, 2, True, "softmax", "normal")
    share = _top1_share(make_logits(w))
    assert share.max() / share.min() < 1.1


def test_zipf_routing_skews_towards_low_ids():
    w = Workload("zipf", 4, 4096, 64, 64, 8, 2, True, "softmax", "zipf", zipf_s=1.2)
    share = _top1_share(make_logits(w))
    # the bias ln p_e orders the experts: expert 0 hottest, shares descending
    assert np.all(np.diff(share) < 0)
    assert share[0] > 3 * share[-1]
    # the bias is exactly ln of the normalised Zipf(1.2) probabilities
    p = zipf_probs(8, 1.2)
    assert p.sum() == pytest.approx(1.0)
    assert p[0] / p[1] == pytest.approx(2 ** 1.2)


def test_layered_routing_varies_per_layer():
    w = WORKLOADS[5].replace(T=256)
    tau = layer_temperatures(w.layers)
    assert tau.shape == (16,) and tau.min() >= 0.5 and tau.max() <= 2.0
    hot = [int(np.argmax(_top1_share(make_logits(w, l)))) for l in range(4)]
    assert len(set(hot)) > 1                              # a different hot expert across layers
    assert not np.array_equal(make_logits(w, 0), make_logits(w, 1))
