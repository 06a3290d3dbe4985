"""moe_expert_forward_noalloc: the expert forward whose GEMM counters and
K-split partial tiles live in the library's static scratch array instead of
the workspace. Through the C ABI it must give the bits of
moe_expert_forward_overlap on the same plan: two calls in a row on two
shapes, the second smaller (the array keeps the first call's counters and
partials), in every mode.
"""
import numpy as np
import pytest

from synth import Workload
from parity_util import bits, make_gpu_share, say

pytestmark = pytest.mark.gpu

# the first shape has split tail tiles in both GEMMs (69 row tiles x 8 column
# tiles of the output projection on 256 CUs); the second is smaller
BIG = Workload("noalloc_big", 4, 2560, 2048, 2048, 16, 2, True, "softmax", "zipf", w_std="fan_in")
SMALL = Workload("noalloc_small", 4, 384, 512, 768, 8, 2, True, "sigmoid", "normal", w_std="fan_in")


def _poison(sh, w):
    b = sh.buf
    b.y_perm.fill_(float("nan"))
    b.h.fill_(float("nan"))
    for q in range(w.R):
        if b.combine[q] is not None:
            b.combine[q].fill_(float("nan"))


def _forward(sh, noalloc, mode, c):
    from combine_overlap_amd import ops
    b = sh.buf
    sh.epoch = (sh.epoch % 0xFFFFFFF0) + 1
    fwd = ops.moe_expert_forward_noalloc if noalloc else ops.moe_expert_forward_overlap
    fwd(sh.ctx, sh.shape, b.x_perm, b.w1, b.w3, b.w2, b.ws, b.h, b.y_perm, b.combine, b.flags, sh.epoch, c, mode)


def _outputs(sh, w, m_pad):
    b = sh.buf
    counts = b.counts.cpu().numpy()
    return (bits(b.y_perm[:m_pad]).copy(),
            {q: bits(b.combine[q][:int(counts[:, q].sum())]).copy() for q in range(w.R) if b.combine[q] is not None},
            bits(b.y_share).copy())


def test_noalloc_matches_overlap_on_two_calls_the_second_smaller():
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL
    shares = []
    for w, tb in ((BIG, 32), (SMALL, 64)):
        say(f"[noalloc] {w.name}: route + permute")
        sh, _ = make_gpu_share(w, 0, tb, 1)
        sh.route()
        sh.permute()
        torch.cuda.synchronize()
        shares.append((w, sh, sh.plan_arrays()["m_pad"]))
    for mode, c in ((MOE_MODE_OVERLAP, 16), (MOE_MODE_ROLE_SWITCH, 16), (MOE_MODE_SEQUENTIAL, 16)):
        refs = []
        for w, sh, m_pad in shares:
            say(f"[noalloc] mode {mode}: {w.name} through moe_expert_forward_overlap")
            _poison(sh, w)
            _forward(sh, False, mode, c)
            sh.combine()
            torch.cuda.synchronize()
            assert sh.status() == 0
            refs.append(_outputs(sh, w, m_pad))
        # the two no-alloc calls back to back, the second on the smaller shape
        for w, sh, m_pad in shares:
            _poison(sh, w)
        for w, sh, m_pad in shares:
            say(f"[noalloc] mode {mode}: {w.name} through moe_expert_forward_noalloc")
            _forward(sh, True, mode, c)
        for w, sh, m_pad in shares:
            sh.combine()
        torch.cuda.synchronize()
        for (w, sh, m_pad), ref in zip(shares, refs):
            assert sh.status() == 0
            got = _outputs(sh, w, m_pad)
            assert np.array_equal(got[0], ref[0]), f"mode {mode} {w.name}: y_perm differs"
            for q in ref[1]:
                assert np.array_equal(got[1][q], ref[1][q]), f"mode {mode} {w.name}: combine buffer {q} differs"
            assert np.array_equal(got[2], ref[2]), f"mode {mode} {w.name}: y_share differs"
