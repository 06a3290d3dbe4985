"""Race and stress tests of the tile-signalling protocol ([TLS] sec. 3.3.1:
store the tile, then raise its flag; the copying roles copy a segment only
once every flag of its row tiles is up).

The publication here is fence-free: device-scope stores, a wait for their
completion, then the flag. These tests perturb when work happens, never what
is computed, so every output must keep the bits of the sequential baseline:
  * seeded per-item delays before each GEMM work item's results go out (the
    tiles finish in a shuffled order, and the chunks of split tail tiles
    arrive far apart);
  * the tile queues walked in reverse schedule order (remote tiles last, so
    the copying roles wait the longest);
  * split tail chunks that never wait for each other (the last chunk of each
    split tile to arrive reduces the whole tile);
plus two exact invariants of the share: scaling W2 by 2 doubles every output
bit-exactly, and permuting the tokens of a rank permutes its outputs
bit-exactly (at a shape without K-split tiles, so every row is summed in the
same order wherever it lands).
"""
import numpy as np
import pytest

from synth import Workload
from parity_util import bits, make_gpu_share, say

pytestmark = pytest.mark.gpu

# many row tiles of several experts and owners, 32-row bands (many segments).
# On 256 CUs this layout has 69 row tiles x 8 column tiles; every XCD queue
# of the output projection ends in tail tiles split 3 ways at c = 16 (30
# producers per XCD) and 4 ways at c = 0 (32 per XCD).
W_RACE = Workload("race_mini", 4, 2560, 2048, 2048, 16, 2, True, "softmax", "zipf", w_std="fan_in")


def _outputs(sh, w, m_pad):
    b = sh.buf
    counts = b.counts.cpu().numpy()
    return (bits(b.y_perm[:m_pad]).copy(),
            {q: bits(b.combine[q][:int(counts[:, q].sum())]).copy() for q in range(w.R) if b.combine[q] is not None},
            bits(b.y_share).copy())


def _poison(sh, w):
    b = sh.buf
    b.y_perm.fill_(float("nan"))
    b.y_share.fill_(float("nan"))
    for q in range(w.R):
        if b.combine[q] is not None:
            b.combine[q].fill_(float("nan"))


def _same(got, want, what):
    assert np.array_equal(got[0], want[0]), f"{what}: y_perm differs"
    for q in want[1]:
        assert np.array_equal(got[1][q], want[1][q]), f"{what}: combine buffer {q} differs"
    assert np.array_equal(got[2], want[2]), f"{what}: y_share differs"


@pytest.mark.parametrize("fused", [False, True])
def test_perturbed_timing_keeps_the_bits(fused):
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL
    w = W_RACE
    sh, _ = make_gpu_share(w, 0, 32, 1)
    sh.fused_gather = fused
    sh.route()
    sh.permute()
    m_pad = sh.plan_arrays()["m_pad"]
    c = 16
    refs = {}
    for c_ref in (c, 0):   # the K-split is sized for n_cu - c: the reference per split
        say(f"[race] fused={fused}: sequential reference, c={c_ref}")
        _poison(sh, w)
        sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=c_ref)
        sh.combine()
        torch.cuda.synchronize()
        assert sh.status() == 0
        refs[c_ref] = _outputs(sh, w, m_pad)
    cases = [("delay seed 1", 1, False, -1), ("delay seed 0x9e37", 0x9E37, False, -1),
             ("reversed schedule", 0, True, -1), ("reversed + delays", 7, True, -1),
             ("tail chunks never wait", 0, False, 0), ("no tail wait + delays", 3, False, 0)]
    for name, seed, rev, tail in cases:
        for mode, mname, ref in ((MOE_MODE_OVERLAP, "cu_partition", refs[c]),
                                 (MOE_MODE_ROLE_SWITCH, "role_switch", refs[0])):
            say(f"[race] fused={fused} {mname}: {name}")
            sh.ctx.set_debug(seed, rev, tail)
            try:
                _poison(sh, w)
                sh.expert_forward(mode, n_consumer_cu=c)
                sh.combine()
                torch.cuda.synchronize()
            finally:
                sh.ctx.set_debug(0, False, -1)
            assert sh.status() == 0, f"{mname} {name}: status {sh.status()}"
            _same(_outputs(sh, w, m_pad), ref, f"{mname} {name}")


def test_doubled_w2_doubles_every_output():
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH
    w = W_RACE
    sh, _ = make_gpu_share(w, 0, 64, 1)
    sh.route()
    sh.permute()
    m_pad = sh.plan_arrays()["m_pad"]
    for mode in (MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH):
        say(f"[race] 2 W2 -> 2 y, mode {mode}")
        base_w2 = sh.buf.w2.clone()
        _poison(sh, w)
        sh.expert_forward(mode, n_consumer_cu=16)
        sh.combine()
        torch.cuda.synchronize()
        y1, b1, s1 = _outputs(sh, w, m_pad)
        sh.buf.w2.copy_((base_w2.float() * 2.0).to(torch.bfloat16))   # exact: a power of two
        try:
            _poison(sh, w)
            sh.expert_forward(mode, n_consumer_cu=16)
            sh.combine()
            torch.cuda.synchronize()
            y2, b2, s2 = _outputs(sh, w, m_pad)
        finally:
            sh.buf.w2.copy_(base_w2)
        assert sh.status() == 0

        def doubled(a):   # bf16 bits of 2x (finite, non-subnormal values: exponent + 1)
            f = (a.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0)
            return (f.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(y2, doubled(y1)), "y_perm"
        for q in b1:
            assert np.array_equal(b2[q], doubled(b1[q])), f"combine buffer {q}"
        assert np.array_equal(s2, doubled(s1)), "y_share"


def test_token_permutation_permutes_outputs():
    """H = 512 and F = 768: the first projection's K = 512 and the output
    projection's K = 768 give at most 12 k-steps, below two chunks of the
    K-split minimum, so no tile is split and every output row is the same
    sequence of fp32 MFMA sums wherever the layout puts it."""
    import torch
    from synth import make_local_weights, make_logits, make_x
    from synth.workloads import ShareInputs
    from combine_overlap_amd import MOE_MODE_OVERLAP
    w = Workload("perm_mini", 4, 768, 512, 768, 16, 4, True, "softmax", "zipf", w_std="fan_in")
    W1, W3, W2 = make_local_weights(w, 1)
    logits, x = make_logits(w, 0), make_x(w)
    rng = np.random.default_rng(11)
    perms = [rng.permutation(w.T) for _ in range(w.R)]
    lg2 = logits.reshape(w.R, w.T, w.E).copy()
    x2 = x.copy()
    for s in range(w.R):
        lg2[s] = lg2[s][perms[s]]
        x2[s] = x2[s][perms[s]]
    outs = []
    for lg, xx in ((logits, x), (lg2.reshape(w.R * w.T, w.E), x2)):
        say(f"[race] token permutation: run {len(outs)}")
        inp = ShareInputs(w, 1, lg, xx, W1, W3, W2)
        sh, _ = make_gpu_share(w, 1, 64, 1, inp)
        sh.layer(MOE_MODE_OVERLAP, n_consumer_cu=8)
        torch.cuda.synchronize()
        assert sh.status() == 0
        outs.append(bits(sh.buf.y_share).reshape(w.R, w.T, w.H).copy())
        del sh
    want = np.stack([outs[0][s][perms[s]] for s in range(w.R)])
    assert np.array_equal(outs[1], want), "y_share is not permuted with the tokens"
