"""Seeded synthetic inputs for one expert-parallel rank's MoE-layer share.

This module only draws random numbers and rounds them to the storage types
(bf16 bit patterns held in uint16, fp32 logits). It holds none of the MoE
method's arithmetic: no routing, no layout, no FFN. Both the CPU oracle's
tests and the GPU path consume the arrays it returns, so the two sides see
identical inputs.

Workloads (shapes follow the five synthetic configurations of the hot path):

=====  =========================================================================
 id    shape
=====  =========================================================================
 1     tiny: R=4 ranks x T=256 tokens, H=512, F=1024, non-gated FFN,
       8 experts (2 local), top-2 softmax gates, logits ~ N(0,1),
       weights ~ N(0, 0.02)
 2     Mixtral-shaped: R=4 x T=4096, H=4096, F=14336, SiLU-gated (W1/W3/W2),
       8 experts (2 local), top-2 softmax, logits ~ N(0,1),
       weights ~ N(0, fan_in^-1/2)
 3     as 2, but logits biased by ln Zipf(s=1.2) over the expert id, so the
       hottest expert (id 0, local to rank 0) gets about 3x the mean load
 4     fine-grained: R=8 x T=2048, H=7168, F=2048 gated, 256 experts (32 local),
       top-8 sigmoid gates normalised over the 8, weights ~ N(0, 0.02)
 5     dynamic split: R=4 x T=8192, H=4096, F=1536 gated, 128 experts
       (32 local), top-8 softmax, 16 layers; layer l has its own logits
       z_l + ln(p[perm_l(e)]) / tau_l with Zipf(1.2) p, a seeded expert
       permutation perm_l and tau_l ~ U(0.5, 2.0); weights ~ N(0, 0.02)
=====  =========================================================================

Every tensor has its own counter-free PCG64 stream keyed by
``(seed, tensor tag, index...)`` so any one expert's weights can be drawn
without drawing the others.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# stream tags
_TAG_LOGITS = 11
_TAG_X = 12
_TAG_W1 = 21
_TAG_W3 = 23
_TAG_W2 = 22
_TAG_LAYER = 31


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one MoE-layer share workload."""

    name: str
    R: int            # simulated ranks
    T: int            # tokens per rank
    H: int            # hidden size
    F: int            # expert FFN width
    E: int            # experts in total (E/R local to each rank)
    k: int            # top-k
    gated: bool       # True: y = (SiLU(x W1^T) * (x W3^T)) W2^T ; False: SiLU(x W1^T) W2^T
    gate_kind: str    # "softmax" or "sigmoid" (normalised over the selected k)
    routing: str = "normal"        # "normal" | "zipf" | "layered"
    zipf_s: float = 1.2
    w_std: str = "0.02"            # "0.02" or "fan_in"
    layers: int = 1
    seed: int = 0

    @property
    def E_local(self) -> int:
        return self.E // self.R

    @property
    def n_tokens(self) -> int:
        return self.R * self.T

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny_r4_t256_h512_f1024_e8_top2", 4, 256, 512, 1024, 8, 2,
                False, "softmax", "normal", w_std="0.02"),
    2: Workload("mixtral_r4_t4096_h4096_f14336_e8_top2", 4, 4096, 4096, 14336, 8, 2,
                True, "softmax", "normal", w_std="fan_in"),
    3: Workload("zipf1.2_r4_t4096_h4096_f14336_e8_top2", 4, 4096, 4096, 14336, 8, 2,
                True, "softmax", "zipf", w_std="fan_in"),
    4: Workload("finegrained_r8_t2048_h7168_f2048_e256_top8", 8, 2048, 7168, 2048, 256, 8,
                True, "sigmoid", "normal", w_std="0.02"),
    5: Workload("dynsplit_r4_t8192_h4096_f1536_e128_top8_x16", 4, 8192, 4096, 1536, 128, 8,
                True, "softmax", "layered", w_std="0.02", layers=16),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(v) for v in key])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even) and return the bit patterns.

    Works in uint32 (no wider temporaries): for finite inputs the rounding
    increment cannot overflow 32 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    r = u.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_probs(E: int, s: float) -> np.ndarray:
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return p / p.sum()


def layer_temperatures(n_layers: int) -> np.ndarray:
    """Per-layer routing temperatures tau_l ~ U(0.5, 2.0) for the layered workload."""
    return _rng(0).uniform(0.5, 2.0, n_layers)


def make_logits(w: Workload, layer: int = 0) -> np.ndarray:
    """Router logits, fp32 [R*T, E], with any bias/temperature already applied."""
    n, E = w.n_tokens, w.E
    if w.routing == "normal":
        return _rng(w.seed, _TAG_LOGITS).standard_normal((n, E), dtype=np.float32)
    if w.routing == "zipf":
        z = _rng(w.seed, _TAG_LOGITS).standard_normal((n, E), dtype=np.float32)
        bias = np.log(zipf_probs(E, w.zipf_s))
        return (z.astype(np.float64) + bias[None, :]).astype(np.float32)
    if w.routing == "layered":
        tau = layer_temperatures(max(w.layers, layer + 1))[layer]
        g = _rng(1000 + layer, _TAG_LAYER)
        perm = g.permutation(E)
        z = _rng(1000 + layer, _TAG_LOGITS).standard_normal((n, E), dtype=np.float32)
        bias = np.log(zipf_probs(E, w.zipf_s))[perm] / tau
        return (z.astype(np.float64) + bias[None, :]).astype(np.float32)
    raise ValueError(f"unknown routing {w.routing!r}")


def make_x(w: Workload) -> np.ndarray:
    """Token activations, bf16 bits [R, T, H], values ~ N(0,1)."""
    g = _rng(w.seed, _TAG_X)
    out = np.empty((w.R, w.T, w.H), dtype=np.uint16)
    for s in range(w.R):  # one rank at a time keeps the fp32 temporary small
        out[s] = f32_to_bf16_bits(g.standard_normal((w.T, w.H), dtype=np.float32))
    return out


def _std(w: Workload, fan_in: int) -> float:
    if w.w_std == "fan_in":
        return float(fan_in) ** -0.5
    return float(w.w_std)


def make_expert_weights(w: Workload, e_glob: int):
    """(W1 [F,H], W3 [F,H] or None, W2 [H,F]) bf16 bits for global expert e_glob.

    Layout follows nn.Linear: [out_features, in_features].
    """
    s1 = _std(w, w.H)
    s2 = _std(w, w.F)
    w1 = f32_to_bf16_bits(_rng(w.seed, _TAG_W1, e_glob).standard_normal((w.F, w.H), dtype=np.float32) * np.float32(s1))
    w3 = None
    if w.gated:
        w3 = f32_to_bf16_bits(_rng(w.seed, _TAG_W3, e_glob).standard_normal((w.F, w.H), dtype=np.float32) * np.float32(s1))
    w2 = f32_to_bf16_bits(_rng(w.seed, _TAG_W2, e_glob).standard_normal((w.H, w.F), dtype=np.float32) * np.float32(s2))
    return w1, w3, w2


def make_local_weights(w: Workload, r_self: int):
    """Stacked weights of rank r_self's local experts: W1/W3 [E_l,F,H], W2 [E_l,H,F].

    Experts are drawn in parallel threads (each has its own stream, so the
    result does not depend on the thread count)."""
    import concurrent.futures as cf
    import os
    El = w.E_local
    W1 = np.empty((El, w.F, w.H), dtype=np.uint16)
    W3 = np.empty((El, w.F, w.H), dtype=np.uint16) if w.gated else None
    W2 = np.empty((El, w.H, w.F), dtype=np.uint16)

    def one(e):
        a, b, c = make_expert_weights(w, r_self * El + e)
        W1[e] = a
        if W3 is not None:
            W3[e] = b
        W2[e] = c

    workers = max(1, min(El, len(os.sched_getaffinity(0)), 16))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(El)))
    return W1, W3, W2


@dataclasses.dataclass
class ShareInputs:
    """All inputs of one rank's share: logits fp32, x / weights as bf16 bits."""

    w: Workload
    r_self: int
    logits: np.ndarray
    x: np.ndarray
    W1: np.ndarray
    W3: Optional[np.ndarray]
    W2: np.ndarray


def make_share_inputs(w: Workload, r_self: int = 0, layer: int = 0) -> ShareInputs:
    W1, W3, W2 = make_local_weights(w, r_self)
    return ShareInputs(w, r_self, make_logits(w, layer), make_x(w), W1, W3, W2)
