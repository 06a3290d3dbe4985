"""A whole layer share captured in a HIP graph and replayed.

route -> permute (the plan also picks the consumer CU count on the device)
-> expert forward with MOE_CONSUMER_AUTO -> combine is one stream of
kernels with no host round trip, so torch.cuda.CUDAGraph can capture it. A
replay reuses the captured epoch; the first projection clears the ready flags
at the start of every call, so no replay can see the previous one's flags.
Every replay must give the eager run's bits (outputs poisoned with NaN in
between, eager work on the side).
"""
import numpy as np
import pytest

from synth import Workload
from parity_util import bits, make_gpu_share, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode_name,fused", [("cu_partition", False), ("cu_partition", True),
                                             ("role_switch", True)])
def test_layer_graph_replay(mode_name, fused):
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH
    mode = {"cu_partition": MOE_MODE_OVERLAP, "role_switch": MOE_MODE_ROLE_SWITCH}[mode_name]
    w = Workload("graph_mini", 4, 512, 1024, 1024, 8, 2, True, "softmax", "zipf", w_std="fan_in")
    say(f"[graph] {mode_name}, fused gather {fused}: capture one layer, replay 3 times")
    sh, _ = make_gpu_share(w, 0, 64, 1)
    sh.fused_gather = fused
    b = sh.buf
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sh.layer(mode)            # eager reference (and warm-up on the capture stream)
    torch.cuda.synchronize()
    assert sh.status() == 0
    m_pad = sh.plan_arrays()["m_pad"]
    ref_share = bits(b.y_share).copy()
    ref_y = bits(b.y_perm[:m_pad]).copy()
    counts = b.counts.cpu().numpy()
    n_recv = {q: int(counts[:, q].sum()) for q in range(w.R)}   # rows the layer writes per buffer
    ref_buf = {q: bits(b.combine[q][:n_recv[q]]).copy() for q in range(w.R) if b.combine[q] is not None}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sh.layer(mode)
    torch.cuda.synchronize()
    for it in range(3):
        b.y_share.fill_(float("nan"))
        b.y_perm.fill_(float("nan"))
        for q in ref_buf:
            b.combine[q].fill_(float("nan"))
        junk = torch.randn(1 << 20, device=b.y_share.device).sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert sh.status() == 0
        assert np.array_equal(bits(b.y_perm[:m_pad]), ref_y), f"replay {it}: y_perm differs"
        for q, r in ref_buf.items():
            assert np.array_equal(bits(b.combine[q][:n_recv[q]]), r), f"replay {it}: combine buffer {q} differs"
        assert np.array_equal(bits(b.y_share), ref_share), f"replay {it}: y_share differs"
        del junk
