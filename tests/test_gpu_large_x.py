"""The gathered first projection with an x of 2 GiB.

Below 2 GiB the gathered rows are loaded through a buffer resource with
32-bit offsets; from 2 GiB on the per-lane 64-bit-address form runs. Here x
is exactly 2 GiB (2 ranks x 65536 tokens x 8192 hidden, bf16), so the second
form runs, and its outputs must equal the materialized path's bit for bit:
y_perm with its padding rows and every combine buffer (the materialized path
itself is checked against the oracle by the other parity tests).
"""
import numpy as np
import pytest

from parity_util import bits, say

pytestmark = pytest.mark.gpu


def test_gathered_projection_with_2gib_x_matches_materialized():
    import torch
    from combine_overlap_amd import MOE_MODE_SEQUENTIAL
    from combine_overlap_amd.share import MoEShare
    R, T, H, F, E, k = 2, 65536, 8192, 128, 4, 1
    assert R * T * H * 2 == 1 << 31
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    say(f"[large x] R={R} T={T} H={H} F={F} E={E} k={k}: x of {R * T * H * 2 / 2**30:.0f} GiB")
    logits = torch.randn((R * T, E), generator=gen, device=dev, dtype=torch.float32)
    x = torch.randn((R, T, H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    El = E // R
    w1 = (torch.randn((El, F, H), generator=gen, device=dev) * H ** -0.5).to(torch.bfloat16)
    w3 = (torch.randn((El, F, H), generator=gen, device=dev) * H ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn((El, H, F), generator=gen, device=dev) * F ** -0.5).to(torch.bfloat16)
    sh = MoEShare(R, T, H, F, E, k, True, "softmax", r_self=0, tb_m=64, device=dev)
    sh.allocate(logits, x, w1, w3, w2)
    b = sh.buf

    sh.fused_gather = False
    sh.route()
    sh.permute()
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=0)
    torch.cuda.synchronize()
    assert sh.status() == 0
    m_pad = sh.plan_arrays()["m_pad"]
    ref_y = bits(b.y_perm[:m_pad]).copy()
    counts = b.counts.cpu().numpy()
    ref_buf = {q: bits(b.combine[q][:int(counts[:, q].sum())]).copy()
               for q in range(R) if b.combine[q] is not None}
    say(f"[large x] materialized: {m_pad} packed rows")

    b.y_perm.fill_(float("nan"))
    for q in ref_buf:
        b.combine[q].fill_(float("nan"))
    b.x_perm = None   # the gathered forward must not need it
    torch.cuda.empty_cache()
    sh.fused_gather = True
    sh.permute()
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=0)
    torch.cuda.synchronize()
    assert sh.status() == 0
    assert np.array_equal(bits(b.y_perm[:m_pad]), ref_y), "gathered y_perm differs from the materialized run"
    for q, r in ref_buf.items():
        assert np.array_equal(bits(b.combine[q][:len(r)]), r), f"combine buffer {q} differs"
