"""The bounded flag wait of the overlapped copy, forced from the host.

With a wait limit of one tick (10 ns of the constant clock) the CU-partition
consumer cannot see its first segment's flags in time (that segment's row
tiles take hundreds of microseconds of the output projection), so it must
give up: the device status word reads MOE_ERR_TIMEOUT, every kernel exits
normally, and the producer's output is the same as an ordinary call's. With
the default limit restored, the next layer runs clean and copies every row.
"""
import numpy as np
import pytest

from synth import Workload
from parity_util import bits, make_gpu_share, say

pytestmark = pytest.mark.gpu


def test_consumer_wait_limit_reports_timeout_and_recovers():
    import torch
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_SEQUENTIAL, _abi
    w = Workload("watchdog_mini", 4, 512, 1024, 2048, 8, 2, True, "softmax", "zipf", w_std="fan_in")
    say("[watchdog] CU partition, c = 16, wait limit 1 tick: expect MOE_ERR_TIMEOUT")
    sh, _ = make_gpu_share(w, 0, 64, 1)
    b = sh.buf
    sh.route()
    sh.permute()
    sh.expert_forward(MOE_MODE_SEQUENTIAL, n_consumer_cu=16)
    torch.cuda.synchronize()
    assert sh.status() == 0
    m_pad = sh.plan_arrays()["m_pad"]
    ref_y = bits(b.y_perm[:m_pad]).copy()
    counts = b.counts.cpu().numpy()
    ref_buf = {q: bits(b.combine[q][:int(counts[:, q].sum())]).copy()
               for q in range(w.R) if b.combine[q] is not None}
    assert sum(len(v) for v in ref_buf.values()) > 0

    sh.ctx.set_wait_limit(1)
    b.y_perm.fill_(float("nan"))
    sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=16)
    torch.cuda.synchronize()
    assert sh.status() == _abi.MOE_ERR_TIMEOUT
    assert np.array_equal(bits(b.y_perm[:m_pad]), ref_y), "producer output changed by the consumer's time-out"

    say("[watchdog] default limit restored: the next layer runs clean")
    sh.ctx.set_wait_limit(0)
    for q in ref_buf:
        b.combine[q].fill_(float("nan"))
    sh.route()
    sh.permute()          # clears the status word
    sh.expert_forward(MOE_MODE_OVERLAP, n_consumer_cu=16)
    torch.cuda.synchronize()
    assert sh.status() == 0
    assert np.array_equal(bits(b.y_perm[:m_pad]), ref_y)
    for q, r in ref_buf.items():
        assert np.array_equal(bits(b.combine[q][:len(r)]), r), f"combine buffer {q}"
