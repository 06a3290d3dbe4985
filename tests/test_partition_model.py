"""The CU-split model against its definition, as events.

moe_plan_partition evaluates the model in a closed form (wave ends from the
maxima of tile times, copy end max_i(ready_i + 2 H S_i / BW)). Here the same
model is restated from its definition and simulated event by event: tile
instances run in waves of P in schedule order, a row tile is ready when the
wave holding its last column tile ends, and the consumer copies the segments
in order, each starting when it is ready and the previous copy is done. The
predicted times must agree to rounding and the chosen c must be the argmin.
"""
import numpy as np
import pytest

from combine_overlap_amd import _abi, ops


def events_model(R, E, H, F, tb, r_self, counts, cal):
    El = E // R
    remote_pad = np.zeros(El, np.int64)
    remote_bands = np.zeros(El, np.int64)
    remote_rows = np.zeros(El, np.int64)
    m_e = np.zeros(El, np.int64)
    for e in range(El):
        for q in range(R):
            c = int(counts[e, q])
            if q == r_self:
                m_e[e] += c
            else:
                nb = -(-c // tb)
                remote_pad[e] += nb * tb
                remote_bands[e] += nb
                remote_rows[e] += c
                m_e[e] += nb * tb
    order = sorted(range(El), key=lambda e: (-remote_bands[e], -remote_rows[e], e))
    alg = [-(-int(m) // tb) * tb for m in m_e]
    rate = [cal.gemm_flops_per_cu * max(int(m), 1) / (max(int(m), 1) + cal.gemm_m_half) for m in m_e]

    def tile_time(e, j):
        rows = min(256, alg[e] - j * 256)
        return 2.0 * (-(-rows // 32) * 32) * 256.0 * F / rate[e]
    # row tiles in schedule order: those reaching into the remote groups (experts
    # in the remote-phase order), then the others by expert id
    sched, pos = [], {}
    for e in order:
        for j in range(-(-int(remote_pad[e]) // 256)):
            pos[(e, j)] = len(sched)
            sched.append((e, j))
    for e in range(El):
        for j in range(-(-int(remote_pad[e]) // 256), -(-alg[e] // 256)):
            pos[(e, j)] = len(sched)
            sched.append((e, j))
    # segments: per (expert, remote owner) group, 1, g, ..., g, (remainder), 1 bands
    g = 2 if 2.0 * tb * H < 0.5 * 1048576.0 else 1
    segs = []   # (valid rows, position of the last band's row tile)
    for e in order:
        rel = 0
        for q in range(R):
            if q == r_self:
                continue
            c = int(counts[e, q])
            nb = -(-c // tb)
            bands = [(min(tb, c - i * tb), rel + i * tb) for i in range(nb)]
            i = 0
            while i < nb:
                sz = 1 if (i == 0 or i == nb - 1) else min(g, nb - 1 - i)
                rows = sum(b[0] for b in bands[i:i + sz])
                last_row = bands[i + sz - 1][1] + tb - 1
                segs.append((rows, pos[(e, last_row // 256)]))
                i += sz
            rel += nb * tb
    tiles2 = -(-H // 256)
    results = {}
    for c in range(cal.c_min, cal.c_max + 1, cal.c_step):
        P = cal.n_cu - c
        inst = [t for t in range(len(sched)) for _ in range(tiles2)]
        ready = [0.0] * len(sched)
        t = 0.0
        for w0 in range(0, len(inst), P):
            wave = inst[w0:w0 + P]
            length = max(tile_time(*sched[x]) for x in wave)
            t += length if len(wave) == P else length * max(len(wave) / P, 1.0 / 3.0)
            for x in set(wave):
                ready[x] = t   # the wave holding a tile's last instance sets it last
        bw = c * cal.copy_bw_per_cu / (1.0 + c * cal.copy_bw_per_cu / cal.copy_bw_max)
        tc = 0.0
        for rows, p in segs:
            tc = max(tc, ready[p]) + 2.0 * rows * H / bw
        results[c] = max(t, tc + cal.seg_latency_s) if segs else t
    return results, g


CASES = [
    # R, E, H, F, k, tb, r_self, counts generator
    (4, 8, 4096, 14336, 2, 64, 0, "uniform"),
    (8, 256, 7168, 2048, 8, 32, 0, "uniform"),
    (4, 128, 4096, 1536, 8, 64, 1, "skew"),
    (4, 16, 8192, 2048, 2, 128, 0, "skew"),
    (2, 4, 2048, 1024, 2, 256, 1, "sparse"),
    (3, 6, 1024, 512, 3, 32, 2, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"R{c[0]}_E{c[1]}_tb{c[5]}_{c[7]}" for c in CASES])
@pytest.mark.parametrize("calib", ["mi355x_like", "halfrate"])
def test_closed_form_matches_event_simulation(case, calib):
    R, E, H, F, k, tb, r_self, kind = case
    El = E // R
    rng = np.random.default_rng(R * 1000 + E + tb)
    if kind == "uniform":
        counts = rng.integers(0, 4 * tb + 7, size=(El, R))
    elif kind == "skew":
        counts = (rng.pareto(1.2, size=(El, R)) * 300).astype(np.int64)
    else:
        counts = rng.integers(0, 3, size=(El, R)) * rng.integers(0, 2000, size=(El, R))
    counts = counts.astype(np.int32)
    if calib == "mi355x_like":
        cal = _abi.MoeCalib(3.5e12, 0.0, 20e9, 800e9, 30e-6, 256, 8, 48, 8)
    else:
        cal = _abi.MoeCalib(2e12, 512.0, 35e9, 2e12, 5e-6, 128, 2, 20, 2)
    sh = ops.make_shape(R, 1 << 14, H, F, E, k, r_self, True, "softmax", tb, 1)
    times, g = events_model(R, E, H, F, tb, r_self, counts, cal)
    c_lib, g_lib, t_lib = ops.moe_plan_partition(sh, counts, cal)
    assert g_lib == g
    best = min(times.values())
    assert t_lib == pytest.approx(best, rel=1e-9)
    assert times[c_lib] == pytest.approx(best, rel=1e-9)   # the argmin (ties to rounding)
    # every candidate: the library's prediction for a one-value range
    for c, t in times.items():
        one = _abi.MoeCalib(cal.gemm_flops_per_cu, cal.gemm_m_half, cal.copy_bw_per_cu, cal.copy_bw_max,
                            cal.seg_latency_s, cal.n_cu, c, c, 1)
        assert ops.moe_plan_partition(sh, counts, one)[2] == pytest.approx(t, rel=1e-9), f"c={c}"
