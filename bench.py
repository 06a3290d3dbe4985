#!/usr/bin/env python3
"""Benchmark: one EP rank's MoE-layer share on one MI355X, overlap vs non-overlap.

A step is one pass of the whole share over one batch of synthetic input:
route -> counts to host -> partition (consumer CUs, segment size) ->
permute -> expert FFN with the overlapped combine transfer -> weighted
reduction. Inputs are resident in HBM before the timed region.

Three forms of the expert phase are timed in the same run: the overlap with
a consumer on its own CU partition (the paper's design), the role-switching
overlap (the producer's workgroups do the copy between tiles), and the
non-overlapped baseline (GEMMs on all CUs, then one bulk copy), each with the
routed rows gathered into x_perm by the permute step and with the gather
fused into the first projection's tile loads. `value` is the fastest
overlapped form (config.overlap_mode, config.gather); the sequential baseline
it is compared with uses the same gather.

Prints ONE JSON line on stdout (details on stderr).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# band height per workload: the fastest measured overlapped layer step
DEFAULT_TB = {1: 64, 2: 64, 3: 256, 4: 32, 5: 64}
# sources whose change invalidates stored hardware-counter traffic figures
GEMM_SOURCES = ("combine_overlap_amd/csrc/gemm.hip", "combine_overlap_amd/csrc/common.hpp",
                "combine_overlap_amd/csrc/consumer.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload id (1-5); 2 = Mixtral-shaped")
    ap.add_argument("--layer", type=int, default=0, help="layer of the layered workload")
    ap.add_argument("--tb", type=int, default=0, help="band height (0 = per-workload default)")
    ap.add_argument("--c", type=int, default=0, help="consumer CUs (0 = cost model)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sequential-only", action="store_true",
                    help="run only the non-overlapped path (for counter collection, which "
                         "serialises kernels and so cannot run the concurrent consumer)")
    ap.add_argument("--gather", choices=("both", "materialized", "fused"), default="both",
                    help="A rows of the first projection: the materialized x_perm, the gather "
                         "fused into its tile loads, or both (timed side by side)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--table2-sweep", action="store_true",
                    help="the shape sweep of the tile-signalling paper's Table 2 on this GPU (tokens per "
                         "rank 8192/16384, K = 2048, N = 4096/8192, experts per rank 4..64, three router "
                         "skews): per shape the sequential baseline, the CU-partition overlap at the "
                         "model's c and at c = 8..48, the other segment size, and role switching; adds a "
                         "'table2_sweep' object to the JSON line")
    ap.add_argument("--layer-sweep", action="store_true",
                    help="layered workload: per layer, the CU-partition overlap at the partition "
                         "model's consumer count and at every candidate count, the role-switching "
                         "overlap and the sequential baseline (expert phase, HIP events); adds a "
                         "'layer_sweep' object to the JSON line")
    return ap.parse_args()


def gemm_source_hash() -> str:
    """16 hex digits of sha256 over the GEMM sources' code: // comments,
    trailing blanks and empty lines are left out, so an edit of comments alone
    keeps the stored counter figures valid."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def stored_figures(name: str):
    """The "- key: value" figures of a committed counter summary under profiles/,
    or None when there is none or the GEMM sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return kv


def stored_traffic(workload: str, tb: int, gathered: bool):
    """HBM-side bytes per launch of the first-projection GEMM from the committed
    FETCH_SIZE / WRITE_SIZE summary for this workload, band height and A-row
    source, or None."""
    kv = stored_figures(f"pmc_gemm1{'_gathered' if gathered else ''}_{workload}_tb{tb}.md")
    try:
        return float(kv["traffic_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def stored_mfma(workload: str, tb: int, gathered: bool):
    """(MFMA-busy fraction of elapsed cycles, running clock in GHz) of the
    first-projection GEMM from the committed counter summary, or None."""
    kv = stored_figures(f"pmc_mfma_{workload}_tb{tb}.md")
    g = "fused" if gathered else "materialized"
    try:
        return (float(kv[f"mfma_busy_gemm1_{g}"]), float(kv[f"clock_ghz_gemm1_{g}"])) if kv else None
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, inp, tb, target_s):
    """Times the CPU oracle (as it is) on a bounded sample of the same workload."""
    from oracle import moe_share as om
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ids, gates = om.route(inp.logits, w.k, w.gate_kind)
    lay = om.row_layout(ids, w.R, w.T, w.E_local, inp.r_self, tb)
    t_route = time.perf_counter() - t0
    # expert FFN on the first n rows of every non-empty local expert
    x_perm = om.gather_rows(inp.x, lay)
    experts = [e for e in range(w.E_local) if lay.M_e[e] > 0]
    wts = {}
    for e in experts:
        wts[e] = (om.widen_bf16(inp.W1[e]), om.widen_bf16(inp.W3[e]) if inp.W3 is not None else None,
                  om.widen_bf16(inp.W2[e]))
    per_row = (6 if w.gated else 4) * w.H * w.F
    n = 8
    flops = 0.0
    t_ffn = 0.0
    while True:
        flops = 0.0
        t0 = time.perf_counter()
        for e in experts:
            lo = int(lay.expert_base[e])
            m = min(n, int(lay.M_e[e]))
            om.expert_ffn(x_perm[lo:lo + m], *wts[e])
            flops += per_row * m
        t_ffn = time.perf_counter() - t0
        if t_ffn >= target_s / 4 or n >= 4096:
            break
        n *= 2
    val = flops / t_ffn / 1e12
    return {"value": round(val, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle: routing+layout of all {w.R * w.T} tokens ({t_route:.2f} s, "
                       f"not in value) and the expert FFN on the first {n} rows of each of "
                       f"{len(experts)} local experts ({flops / 1e9:.1f} GFLOP in {t_ffn:.2f} s)")}


def hbm_phases(sh, w, torch, M, m_pad, remote, bulk_copy_ms, reps=20):
    """The HBM-bound steps timed alone (HIP events on the stream they run on),
    each against the 8 TB/s HBM peak with its algorithmic bytes per launch:
    route (logits read, ids and gates written), the gather into x_perm (valid
    rows read, padded rows written), combine (the local rows read once, the
    share written) and the baseline's bulk copy (remote rows read and written)."""
    s = torch.cuda.current_stream()
    RT, H = w.R * w.T, w.H
    b_route = RT * (4 * w.E + 8 * w.k)
    b_gather = 2 * H * (M + m_pad) + 4 * (RT * w.k + m_pad)
    b_combine = 2 * H * (M + RT) + 12 * RT * w.k
    b_bulk = 4 * H * remote

    def time_it(fn):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(s)
            fn()
            b.record(s)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))
    fused = sh.fused_gather
    sh.fused_gather = False
    out = {}
    for name, fn, nbytes in (("route", lambda: sh.route(s), b_route),
                             ("permute_materialized", lambda: sh.permute(s), b_gather),
                             ("combine", lambda: sh.combine(s), b_combine)):
        out[name] = {"us": time_it(fn) * 1e3, "bytes": nbytes}
    sh.fused_gather = fused
    sh.permute(s)
    out["bulk_copy"] = {"us": bulk_copy_ms * 1e3, "bytes": b_bulk}
    for d in out.values():
        gbs = d["bytes"] / (d["us"] * 1e-6) / 1e9
        d.update({"us": round(d["us"], 2), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)})
    return out


def layer_sweep(sh, w, make_logits, torch, ops, modes, reps=5, cands=(8, 16, 24, 32, 40, 48)):
    """Expert-phase times (ms, median of reps after 2 warmups) per layer and form.

    Compares the partition model's per-layer consumer count with the best
    single count over all layers and with the best count of each layer."""
    MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL = modes
    sh.ctx.set_timing(True)

    def phase(mode, c):
        d = []
        for i in range(reps + 2):
            sh.expert_forward(mode, n_consumer_cu=c)
            if i >= 2:
                d.append(sh.ctx.timings()["total"])
        return float(np.median(d))
    rows = []
    for layer in range(w.layers):
        sh.buf.logits.copy_(torch.from_numpy(make_logits(w, layer)))
        sh.route()
        sh.permute()
        torch.cuda.synchronize()
        counts = sh.buf.counts.cpu().numpy()
        c_model, _, pred = ops.moe_plan_partition(sh.shape, counts)
        t = {c: phase(MOE_MODE_OVERLAP, c) for c in cands}
        if c_model not in t:
            t[c_model] = phase(MOE_MODE_OVERLAP, c_model)
        row = {"layer": layer, "valid_rows": int(counts.sum()), "counts": counts.tolist(),
               "remote_rows": int(counts.sum() - counts[:, sh.r_self].sum()),
               "c_model": int(c_model), "predicted_ms": round(pred * 1e3, 4),
               "partition_ms": {str(c): round(v, 4) for c, v in sorted(t.items())},
               "role_switch_ms": round(phase(MOE_MODE_ROLE_SWITCH, c_model), 4),
               "sequential_ms": round(phase(MOE_MODE_SEQUENTIAL, c_model), 4)}
        rows.append(row)
        log(f"[sweep] layer {layer:2d}: rows {row['valid_rows']}, model c={c_model} "
            f"{t[c_model]:.3f} ms, best c={min(cands, key=t.get)} {min(t[c] for c in cands):.3f} ms, "
            f"role switch {row['role_switch_ms']:.3f}, sequential {row['sequential_ms']:.3f}")
    sh.ctx.set_timing(False)
    tot = lambda f: round(sum(f(r) for r in rows), 4)
    fixed = {c: tot(lambda r, c=c: r["partition_ms"][str(c)]) for c in cands}
    c_fixed = min(fixed, key=fixed.get)
    return {"layers": rows,
            "total_ms": {"model_c": tot(lambda r: r["partition_ms"][str(r["c_model"])]),
                         "best_fixed_c": fixed[c_fixed], "best_fixed_c_value": c_fixed,
                         "per_layer_best_c": tot(lambda r: min(r["partition_ms"][str(c)] for c in cands)),
                         "role_switch": tot(lambda r: r["role_switch_ms"]),
                         "sequential": tot(lambda r: r["sequential_ms"])}}


# Table 2 of the tile-signalling paper: shape grid of its overlap-vs-baseline
# study. Its expert GEMM (K = 2048 -> N) is the output projection that
# raises the flags, so a shape is a non-gated FFN with F = K and H = N.
# Router modes (named, not defined on the pages): balanced = unbiased logits,
# moderate / stress = logits biased by ln Zipf(s) over the expert id with
# s = 0.6 / 1.2 (the hottest experts local to the timed rank).
TABLE2_SKEWS = (("balanced", "normal", 0.0), ("moderate_skew", "zipf", 0.6), ("stress_skew", "zipf", 1.2))


def table2_sweep(args, torch, reps=5):
    from synth import Workload, make_logits
    from combine_overlap_amd import (MOE_CONSUMER_AUTO, MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH,
                                     MOE_MODE_SEQUENTIAL)
    from combine_overlap_amd.share import MoEShare
    dev = torch.device("cuda:0")
    R, K, topk, tb = 4, 2048, 2, 64
    Ns = (8192, 4096)
    rows = []
    for N in Ns:
        for E_l in (4, 8, 16, 32, 64):
            # activations and weights from a seeded device generator (timing only:
            # no oracle reads them); std 0.02 as for the other small-std workloads
            gen = torch.Generator(device=dev)
            gen.manual_seed(2000 + N + E_l)
            w1 = (torch.randn((E_l, K, N), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            w2 = (torch.randn((E_l, N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            for tpr in (8192, 16384):
                x = torch.randn((R, tpr, N), generator=gen, device=dev).to(torch.bfloat16)
                for skew, routing, zs in TABLE2_SKEWS:
                    w = Workload(f"table2_{skew}_tpr{tpr}_n{N}_e{E_l}", R, tpr, N, K, R * E_l, topk, False,
                                 "softmax", routing, zipf_s=zs or 1.2)
                    sh = MoEShare(R, tpr, N, K, R * E_l, topk, False, "softmax", r_self=0, tb_m=tb,
                                  device=dev, fused_gather=True)
                    sh.allocate(torch.from_numpy(make_logits(w, 0)).to(dev), x, w1, None, w2)
                    for _ in range(2):
                        sh.layer(MOE_MODE_OVERLAP)
                    torch.cuda.synchronize()
                    if sh.status() != 0:
                        raise RuntimeError(f"{w.name}: device status {sh.status()}")
                    c_model, pred = sh.auto_consumer_cu()
                    counts = sh.buf.counts.cpu().numpy()
                    M = int(counts.sum())
                    remote = int(M - counts[:, 0].sum())

                    # layer steps: blocks of `reps` back-to-back steps, the forms taken in
                    # turn over 3 rounds, median block per form
                    forms = (("sequential", MOE_MODE_SEQUENTIAL), ("cu_partition", MOE_MODE_OVERLAP),
                             ("role_switch", MOE_MODE_ROLE_SWITCH))
                    blocks = {m: [] for m, _ in forms}
                    for _ in range(3):
                        for m, v in forms:
                            torch.cuda.synchronize()
                            t0 = time.perf_counter()
                            for _ in range(reps):
                                sh.layer(v)
                            torch.cuda.synchronize()
                            blocks[m].append((time.perf_counter() - t0) / reps * 1e3)
                    layer = {m: float(np.median(b)) for m, b in blocks.items()}
                    sh.ctx.set_timing(True)

                    def phase(mode, c):   # (operator = output projection + transfer, expert phase, exposed)
                        d = []
                        for i in range(reps + 2):
                            sh.expert_forward(mode, n_consumer_cu=c)
                            if i >= 2:
                                d.append(sh.ctx.timings())
                        return tuple(float(np.median([t[k] for t in d]))
                                     for k in ("producer_start_to_consumer_end", "total", "exposed"))
                    seq = phase(MOE_MODE_SEQUENTIAL, MOE_CONSUMER_AUTO)
                    rs = phase(MOE_MODE_ROLE_SWITCH, MOE_CONSUMER_AUTO)
                    by_c = {c: phase(MOE_MODE_OVERLAP, c) for c in (8, 16, 24, 32, 40, 48)}
                    mgb0 = sh.shape.mgb
                    sh.set_routing(mgb=3 - mgb0)   # the other segment size, same c
                    sh.permute()
                    alt = phase(MOE_MODE_OVERLAP, c_model)
                    sh.set_routing(mgb=mgb0)
                    sh.permute()
                    sh.ctx.set_timing(False)
                    ovl = by_c[c_model]
                    c_best = min(by_c, key=lambda c: by_c[c][0])
                    row = {"N": N, "E": E_l, "tpr": tpr, "router": skew, "valid_rows": M, "remote_rows": remote,
                           "c_model": c_model, "c_best": c_best, "mgb": mgb0, "counts": counts.tolist(),
                           "operator_ms": {"sequential": round(seq[0], 4), "cu_partition": round(ovl[0], 4),
                                           "cu_partition_best_c": round(by_c[c_best][0], 4),
                                           "cu_partition_other_mgb": round(alt[0], 4),
                                           "role_switch": round(rs[0], 4)},
                           "expert_phase_ms": {"sequential": round(seq[1], 4), "cu_partition": round(ovl[1], 4),
                                               "role_switch": round(rs[1], 4)},
                           "operator_ms_by_c": {str(c): round(v[0], 4) for c, v in by_c.items()},
                           "layer_ms": {k: round(v, 4) for k, v in layer.items()},
                           "operator_speedup": round(seq[0] / ovl[0], 4),
                           "layer_speedup": round(layer["sequential"] / layer["cu_partition"], 4),
                           "overlap_ratio": round(1.0 - min(1.0, ovl[2] / seq[2]), 4) if seq[2] > 0 else None}
                    rows.append(row)
                    log(f"[table2] N={N} E={E_l} tpr={tpr} {skew}: rows {M} (remote {remote}), c model "
                        f"{c_model} / best {c_best}; operator seq {seq[0]:.3f} ovl {ovl[0]:.3f} "
                        f"rs {rs[0]:.3f} ms; layer seq {layer['sequential']:.3f} ovl "
                        f"{layer['cu_partition']:.3f} rs {layer['role_switch']:.3f} ms; overlap ratio "
                        f"{row['overlap_ratio']}")
                    del sh
                    torch.cuda.empty_cache()
            del w1, w2
            torch.cuda.empty_cache()
    return {"reading": "expert GEMM = output projection of a non-gated FFN, F = K = 2048, H = N; R = 4, "
                       "top-2 softmax; gather fused; router modes as TABLE2_SKEWS",
            "configs": rows}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only (this build runs on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    from synth import WORKLOADS, make_logits, make_x, make_local_weights
    from synth.workloads import ShareInputs
    from combine_overlap_amd import MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL
    from combine_overlap_amd.share import MoEShare, bf16_tensor
    from combine_overlap_amd import ops

    w = WORKLOADS[args.config]
    tb = args.tb or DEFAULT_TB[args.config]
    r_self = 0
    log(f"[bench] workload {w.name} layer {args.layer} tb_m={tb}: generating inputs")
    W1, W3, W2 = make_local_weights(w, r_self)
    inp = ShareInputs(w, r_self, make_logits(w, args.layer), make_x(w), W1, W3, W2)
    dev = torch.device("cuda:0")
    sh = MoEShare(w.R, w.T, w.H, w.F, w.E, w.k, w.gated, w.gate_kind, r_self=r_self, tb_m=tb,
                  device=dev)
    sh.allocate(torch.from_numpy(inp.logits).to(dev), bf16_tensor(inp.x, dev), bf16_tensor(W1, dev),
                bf16_tensor(W3, dev) if W3 is not None else None, bf16_tensor(W2, dev))
    torch.cuda.synchronize()
    n_cu = sh.ctx.num_cus
    log(f"[bench] device CUs {n_cu}; buffers ready")

    def step(mode):
        sh.layer(mode, n_consumer_cu=args.c or None)

    gathers = {"both": (False, True), "materialized": (False,), "fused": (True,)}[args.gather]
    sh.fused_gather = gathers[0]
    main_mode = MOE_MODE_SEQUENTIAL if args.sequential_only else MOE_MODE_OVERLAP
    # warmup + sanity
    for _ in range(max(1, args.warmup)):
        step(main_mode)
    torch.cuda.synchronize()
    if sh.status() != 0:
        raise RuntimeError(f"device status {sh.status()} after warmup")
    # consumer CUs: the plan kernel's choice (no host round trip in the step)
    c_used = args.c or sh.auto_consumer_cu()[0]
    mgb_used = sh.shape.mgb
    counts = sh.buf.counts.cpu().numpy()
    M = int(counts.sum())
    remote = int(counts.sum() - counts[:, r_self].sum())
    per_row = (6 if w.gated else 4) * w.H * w.F
    flops = float(per_row) * M
    flops1 = float((4 if w.gated else 2) * w.H * w.F) * M
    plan = sh.plan_arrays()
    m_pad = plan["m_pad"]
    # compulsory HBM bytes of the first-projection GEMM: its A rows (x_perm, or
    # the valid rows of x when gathered: padding reads one cached zero row),
    # W1 (+W3) of the experts that received rows, h
    n_w = (2 if w.gated else 1) * int((counts.sum(axis=1) > 0).sum())
    gemm1_bytes = {False: 2 * (m_pad * w.H + n_w * w.F * w.H + m_pad * w.F),
                   True: 2 * (M * w.H + n_w * w.F * w.H + m_pad * w.F)}
    log(f"[bench] valid rows {M}, remote rows {remote}, padded rows {m_pad}, bands {plan['n_bands']}, "
        f"segments {plan['n_seg']}, c={c_used}, mgb={mgb_used}")
    log(f"[bench] first-projection algorithmic bytes: materialized {gemm1_bytes[False]}, "
        f"fused {gemm1_bytes[True]}")

    def timed(mode, k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            step(mode)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / k

    modes = ((MOE_MODE_SEQUENTIAL,) if args.sequential_only else
             (MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL))
    mname = {MOE_MODE_OVERLAP: "cu_partition", MOE_MODE_ROLE_SWITCH: "role_switch",
             MOE_MODE_SEQUENTIAL: "sequential"}
    gname = {False: "materialized", True: "fused"}
    t_step = {}
    for fused in gathers:
        sh.fused_gather = fused
        for mode in modes:
            for _ in range(args.warmup):
                step(mode)
            t_step[(fused, mode)] = timed(mode, args.steps)
            log(f"[bench] gather {gname[fused]}, {mname[mode]}: layer step "
                f"{t_step[(fused, mode)] * 1e3:.3f} ms")

    # per-phase device timings (HIP events on the kernels' own streams)
    sh.ctx.set_timing(True)
    ph = {}
    for fused in gathers:
        sh.fused_gather = fused
        sh.permute()
        for mode in modes:
            ph[(fused, mode)] = []
            for _ in range(max(3, args.steps)):
                sh.expert_forward(mode, n_consumer_cu=c_used)
                ph[(fused, mode)].append(sh.ctx.timings())
    sh.ctx.set_timing(False)
    torch.cuda.synchronize()
    if sh.status() != 0:
        raise RuntimeError(f"device status {sh.status()} after the timed runs")

    def med(fused, mode, key):
        return float(np.median([d[key] for d in ph[(fused, mode)]]))
    for fused in gathers:
        log(f"[bench] gather {gname[fused]}, sequential: gemm1 {med(fused, MOE_MODE_SEQUENTIAL, 'gemm1'):.3f} ms, "
            f"gemm2 {med(fused, MOE_MODE_SEQUENTIAL, 'producer'):.3f} ms, bulk copy "
            f"{med(fused, MOE_MODE_SEQUENTIAL, 'exposed') * 1e3:.1f} us, expert phase "
            f"{med(fused, MOE_MODE_SEQUENTIAL, 'total'):.3f} ms")
        if not args.sequential_only:
            log(f"[bench] gather {gname[fused]}, overlap: gemm1 {med(fused, MOE_MODE_OVERLAP, 'gemm1'):.3f} ms, "
                f"output projection + consumer {med(fused, MOE_MODE_OVERLAP, 'producer'):.3f} ms, expert phase "
                f"{med(fused, MOE_MODE_OVERLAP, 'total'):.3f} ms, exposed copy "
                f"{med(fused, MOE_MODE_OVERLAP, 'exposed') * 1e3:.1f} us; role switch: expert phase "
                f"{med(fused, MOE_MODE_ROLE_SWITCH, 'total'):.3f} ms")
    overlapped = [k for k in t_step if k[1] != MOE_MODE_SEQUENTIAL] or list(t_step)
    best = min(overlapped, key=t_step.get)
    b_fused, b_mode = best
    t_best = t_step[best]
    t_seq = t_step[(b_fused, MOE_MODE_SEQUENTIAL)]
    g1 = med(b_fused, b_mode, "gemm1")
    ach1 = flops1 / (g1 * 1e-3) / 1e12
    traffic = stored_traffic(w.name, tb, b_fused)
    mfma = stored_mfma(w.name, tb, b_fused)

    hbm = hbm_phases(sh, w, torch, M, m_pad, remote, med(b_fused, MOE_MODE_SEQUENTIAL, "exposed"))
    log("[bench] HBM-bound steps: " + ", ".join(f"{k} {v['us']:.1f} us {v['GB/s']:.0f} GB/s ({v['frac']:.2f})"
                                                for k, v in hbm.items()))
    layer = {
        "valid_rows": M, "remote_rows": remote, "padded_rows": m_pad,
        "algorithmic_tflop": round(flops / 1e12, 4),
        "step_ms": {gname[f]: {mname[m]: round(t_step[(f, m)] * 1e3, 4) for m in modes} for f in gathers},
        "sequential_ms": round(t_seq * 1e3, 4),
        "speedup_vs_sequential": round(t_seq / t_best, 4),
        "gemm1_ms": round(g1, 4),
    }
    for fused in gathers:
        seq_copy = med(fused, MOE_MODE_SEQUENTIAL, "exposed")
        d = {"sequential": {"expert_phase_ms": round(med(fused, MOE_MODE_SEQUENTIAL, "total"), 4),
                            "gemm1_ms": round(med(fused, MOE_MODE_SEQUENTIAL, "gemm1"), 4),
                            "gemm2_ms": round(med(fused, MOE_MODE_SEQUENTIAL, "producer"), 4),
                            "bulk_copy_us": round(seq_copy * 1e3, 2)}}
        if not args.sequential_only:
            # one launch holds both roles: the producer ends where the exposed copy begins
            launch = med(fused, MOE_MODE_OVERLAP, "producer")
            exposed = med(fused, MOE_MODE_OVERLAP, "exposed")
            prod = launch - exposed
            d["cu_partition"] = {
                "consumer_cus": c_used, "expert_phase_ms": round(med(fused, MOE_MODE_OVERLAP, "total"), 4),
                "gemm1_ms": round(med(fused, MOE_MODE_OVERLAP, "gemm1"), 4),
                "output_projection_launch_ms": round(launch, 4),
                "producer_ms": round(prod, 4),
                "producer_tflops": round(float(2 * w.H * w.F * M) / (prod * 1e-3) / 1e12, 2),
                "exposed_copy_us": round(exposed * 1e3, 2),
                "exposed_copy_fraction": round(exposed / seq_copy, 4) if seq_copy > 0 else None}
            d["role_switch"] = {"expert_phase_ms": round(med(fused, MOE_MODE_ROLE_SWITCH, "total"), 4),
                                "gemm2_and_copy_ms": round(med(fused, MOE_MODE_ROLE_SWITCH, "producer"), 4)}
        layer["gather_" + gname[fused]] = d
    if not args.sequential_only:
        layer["pct_mfma_peak_layer"] = round(100 * flops / t_best / 1e12 / PEAK_BF16_TFLOPS, 2)
    out = {
        "metric": "MoE-layer time/TFLOP/s per EP rank (overlap vs non-overlap), % MFMA peak",
        "value": round(flops / t_best / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_best * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": w.name, "layer": args.layer, "R": w.R, "T": w.T, "H": w.H, "F": w.F,
                   "E": w.E, "k": w.k, "r_self": r_self, "tb_m": tb, "overlap_mode": mname[b_mode],
                   "gather": gname[b_fused],
                   "consumer_cus": c_used, "mgb": mgb_used,
                   "parallelism": "one EP rank share on one GPU"},
        "layer": layer,
        "hbm_kernels": hbm,
        "roofline": {"kernel": "k_gemm first projection (x W1^T, x W3^T, SiLU gate)" +
                     (", rows gathered from x" if b_fused else ""),
                     "bound": "mfma", "achieved": round(ach1, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach1 / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": gemm1_bytes[b_fused], "launch_ms": round(g1, 4),
                     # hardware counters of the same kernel (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE):
                     # the clock it runs at under load and the share of those cycles the matrix
                     # cores are busy; frac_at_running_clock prices achieved against that clock
                     "mfma_busy_pmc": mfma[0] if mfma else None,
                     "clock_ghz_pmc": mfma[1] if mfma else None,
                     "frac_at_running_clock": (round(ach1 / (PEAK_BF16_TFLOPS * mfma[1] / 2.4), 4)
                                               if mfma else None)},
    }
    if args.layer_sweep and w.layers > 1:
        log(f"[bench] layer sweep (gather {gname[b_fused]})")
        sh.fused_gather = b_fused
        out["layer_sweep"] = layer_sweep(sh, w, make_logits, torch, ops,
                                         (MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL))
        log("[bench] layer sweep totals " + json.dumps(out["layer_sweep"]["total_ms"]))
    if args.table2_sweep:
        log("[bench] Table-2 sweep")
        del sh
        torch.cuda.empty_cache()
        out["table2_sweep"] = table2_sweep(args, torch)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, inp, tb, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
