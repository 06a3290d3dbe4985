"""Plain, slow CPU oracle for one expert-parallel rank's MoE-layer share.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module. It shares no
code with the HIP path (no kernels, headers, helpers or table generators);
the only thing the two sides have in common is the seeded input arrays.

Source: "Fine-grained Computation-Communication Overlap via Tile-level
Signaling and Scheduling for Mixture-of-Experts" (arXiv 2607.19539), cited
below as [TLS] with the section, algorithm or table. Floating point is fp64
throughout; bf16 inputs are widened exactly. Nothing is rounded inside.

Notation (follows [TLS] sec. 3.2 and Algorithm 1):
  R ranks, T tokens per rank, H hidden, F expert FFN width, E experts in
  total, E_l = E/R local experts (rank r owns global experts
  [r*E_l, (r+1)*E_l)), top-k, r_self the rank whose share is computed,
  tb_m the tile height in M (one "row band"), mgb = x the number of row
  bands in a middle transfer segment.

Readings of points the pages leave open are stated where they are used
(top-k tie-break, gate normalisation, row order inside a group, group order,
expert sort keys, expert placement, segment scope, receive-buffer layout).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np


# --------------------------------------------------------------------------
# helpers private to the oracle
# --------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


# --------------------------------------------------------------------------
# step 1: routing  ([TLS] sec. 2.1, step 1 "Routing"; MoE definition in 2.1)
# --------------------------------------------------------------------------

def route(logits: np.ndarray, k: int, gate_kind: str):
    """Top-k expert ids and gate weights per token.

    [TLS] sec. 2.1: the router picks the top-k experts of a probability
    distribution; the layer output is the gate-weighted sum of their outputs.

    Readings: selection is on the raw fp32 logits (softmax and sigmoid are
    monotone, so they select the same set); order is highest logit first and
    equal logits go to the lower expert id (a stable sort of -logit). Gates:
      softmax: g_j = exp(l_j - l_1) / sum_i exp(l_i - l_1) over the k selected
      sigmoid: g_j = sigma(l_j) / sum_i sigma(l_i) over the k selected
    so the gates of a token sum to 1.

    Returns ids int32 [N, k] (global expert ids) and gates float64 [N, k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    if gate_kind == "softmax":
        z = np.exp(sel - sel[:, :1])
        gates = z / z.sum(axis=1, keepdims=True)
    elif gate_kind == "sigmoid":
        sg = 1.0 / (1.0 + np.exp(-sel))
        gates = sg / sg.sum(axis=1, keepdims=True)
    else:
        raise ValueError(gate_kind)
    return ids, gates


# --------------------------------------------------------------------------
# step 2: histogram of rows per (local expert, source rank)
# --------------------------------------------------------------------------

def local_histogram(ids: np.ndarray, R: int, T: int, E_l: int, r_self: int) -> np.ndarray:
    """count[e][s] = number of (token of rank s, slot j) routed to local expert e.

    [TLS] Algorithm 1: G_r = rows from rank r routed to local expert e; the
    dispatch (sec. 2.1 step 2) delivers exactly these rows to rank r_self.
    """
    counts = np.zeros((E_l, R), dtype=np.int64)
    first = r_self * E_l
    for s in range(R):
        blk = ids[s * T:(s + 1) * T]
        for e in range(E_l):
            counts[e, s] = int(np.count_nonzero(blk == first + e))
    return counts


# --------------------------------------------------------------------------
# step 3: remote-owner-aligned row layout  ([TLS] sec. 3.2.1, Algorithm 1)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Layout:
    R: int
    T: int
    E_l: int
    r_self: int
    tb_m: int
    counts: np.ndarray        # [E_l, R] valid rows per group
    padded: np.ndarray        # [E_l, R] rows per group incl. zero padding
    group_order: List[int]    # group order inside each expert: remote ranks asc, then r_self
    group_row: np.ndarray     # [E_l, R] absolute first row of group (e, s)
    M_e: np.ndarray           # [E_l] rows of X_e (remote groups padded, local group not)
    expert_base: np.ndarray   # [E_l + 1] first row of X_e in the packed buffer
    m_pad: int                # rows of the packed buffer
    row_src: Optional[np.ndarray]   # [m_pad] global token index s*T+t of each row, -1 for zero rows
    recv_off: np.ndarray      # [R, E_l] first row of (e, s) in rank s's receive buffer
    recv_rows: np.ndarray     # [R] rows of rank s's receive buffer from this rank
    recv_row: Optional[np.ndarray]  # [R*T, k] where slot j of token g is found, -1 if not local


def group_order(R: int, r_self: int) -> List[int]:
    """Reading of [TLS] Algorithm 1 "append G_0..G_{R-1} (remote first, G_self last)":
    the remote groups in ascending rank order, skipping r_self, then G_self."""
    return [s for s in range(R) if s != r_self] + [r_self]


def counts_layout(counts: np.ndarray, R: int, T: int, E_l: int, r_self: int, tb_m: int) -> Layout:
    """The parts of the row layout that follow from the counts alone ([TLS]
    sec. 3.2.1, Algorithm 1): padded group sizes, group and expert offsets,
    receive offsets. row_src and recv_row are left as None (row_layout fills
    them from the routing).

    For each local expert: owner groups in the order of group_order, a remote
    group whose size is not a multiple of tb_m padded with zero rows up to the
    next multiple, the local group not padded.

    Placement reading: [TLS] sec. 3.2 keeps a separate A matrix per expert;
    here X_e sits in one packed buffer at expert_base[e], the exclusive prefix
    sum of M_e rounded up to tb_m, so every row band starts tile-aligned. Rows
    between the end of X_e and the next base belong to no expert and are zero.

    The receive-buffer reading ([TLS] sec. 3.2.3 fixes only that placements do
    not overlap): rank s's buffer holds this rank's rows for s ordered by
    (local expert, token), so recv_off[s][e] = sum_{e' < e} count[e'][s].
    """
    counts = np.asarray(counts, dtype=np.int64).reshape(E_l, R)
    order = group_order(R, r_self)
    padded = counts.copy()
    for e in range(E_l):
        for s in range(R):
            if s != r_self and counts[e, s] % tb_m != 0:
                padded[e, s] = _ceil_div(counts[e, s], tb_m) * tb_m
    M_e = padded.sum(axis=1)
    expert_base = np.zeros(E_l + 1, dtype=np.int64)
    for e in range(E_l):
        expert_base[e + 1] = expert_base[e] + _ceil_div(M_e[e], tb_m) * tb_m
    m_pad = int(expert_base[E_l])

    group_row = np.zeros((E_l, R), dtype=np.int64)
    for e in range(E_l):
        r = int(expert_base[e])
        for s in order:
            group_row[e, s] = r
            r += int(padded[e, s])

    recv_off = np.zeros((R, E_l), dtype=np.int64)
    for s in range(R):
        acc = 0
        for e in range(E_l):
            recv_off[s, e] = acc
            acc += int(counts[e, s])
    recv_rows = counts.sum(axis=0)
    return Layout(R, T, E_l, r_self, tb_m, counts, padded, order, group_row, M_e,
                  expert_base, m_pad, None, recv_off, recv_rows, None)


def row_layout(ids: np.ndarray, R: int, T: int, E_l: int, r_self: int, tb_m: int) -> Layout:
    """Build the per-expert row layouts X_e of [TLS] sec. 3.2.1 / Algorithm 1.

    The group sizes, padding and offsets are those of counts_layout for the
    histogram of the routing. Rows inside a group keep the ascending token
    order of the owner rank (reading: a stable counting sort); row_src maps
    every packed row to its token (-1 for zero rows) and recv_row maps every
    local (token, slot) to where its expert row is found: the combine-buffer
    row for a remote owner, the packed row for r_self.
    """
    lay = counts_layout(local_histogram(ids, R, T, E_l, r_self), R, T, E_l, r_self, tb_m)
    k = ids.shape[1]
    row_src = np.full(lay.m_pad, -1, dtype=np.int64)
    recv_row = np.full((R * T, k), -1, dtype=np.int64)
    first = r_self * E_l
    for e in range(E_l):
        for s in lay.group_order:
            blk = ids[s * T:(s + 1) * T] == first + e          # [T, k]
            toks = np.nonzero(blk.any(axis=1))[0]              # ascending t
            slots = np.argmax(blk[toks], axis=1)               # the one slot holding e
            rows = int(lay.group_row[e, s]) + np.arange(toks.size)
            g = s * T + toks
            row_src[rows] = g
            if s == r_self:
                recv_row[g, slots] = rows
            else:
                recv_row[g, slots] = int(lay.recv_off[s, e]) + np.arange(toks.size)
    lay.row_src = row_src
    lay.recv_row = recv_row
    return lay


def gather_rows(x_bits: np.ndarray, lay: Layout) -> np.ndarray:
    """The packed GEMM input: row i = x of token row_src[i], zero for padding.

    [TLS] sec. 2.1 step 2 (the dispatch delivers the tokens) and sec. 3.2.1
    (zero-filled padding rows). Returns float64 [m_pad, H].
    """
    R, T, H = x_bits.shape
    flat = widen_bf16(x_bits.reshape(R * T, H))
    out = np.zeros((lay.m_pad, H), dtype=np.float64)
    ok = lay.row_src >= 0
    out[ok] = flat[lay.row_src[ok]]
    return out


# --------------------------------------------------------------------------
# step 4: remote-first tile schedule and combine plan
#         ([TLS] sec. 3.2.2, Algorithm 1; sec. 3.2.3)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Bands:
    """Row bands in schedule order. A band is tb_m rows x the full output width;
    its column tiles run in ascending order inside the band ([TLS] sec. 3.2.2)."""

    expert: np.ndarray    # local expert of the band
    row0: np.ndarray      # first row in the packed buffer
    dest: np.ndarray      # owner rank of the band's rows (r_self for local bands)
    recv0: np.ndarray     # first row in dest's receive buffer (-1 for local bands)
    valid: np.ndarray     # non-padding rows of the band
    n_remote: int         # the first n_remote bands are remote-publishable


def tile_schedule(lay: Layout) -> Bands:
    """Remote-first band schedule of [TLS] sec. 3.2.2 / Algorithm 1 plus the
    per-band combine plan of sec. 3.2.3 (destination, receive offset, valid rows).

    Rule (i): every remote band precedes every local band.
    Rule (ii), reading: experts are ordered by remote row-band count
    (descending), ties by remote valid rows (descending), then by expert id.
    Each expert's remote bands stay contiguous, in layout order. Local bands
    follow in expert-id order.
    """
    E_l, R, r_self, tb = lay.E_l, lay.R, lay.r_self, lay.tb_m
    remote = [s for s in lay.group_order if s != r_self]
    n_rb = np.array([sum(_ceil_div(lay.counts[e, s], tb) for s in remote) for e in range(E_l)])
    n_rr = np.array([sum(int(lay.counts[e, s]) for s in remote) for e in range(E_l)])
    expert_order = sorted(range(E_l), key=lambda e: (-int(n_rb[e]), -int(n_rr[e]), e))

    ex, r0, de, rc, va = [], [], [], [], []
    for e in expert_order:
        for s in remote:
            c = int(lay.counts[e, s])
            for i in range(_ceil_div(c, tb)):
                ex.append(e)
                r0.append(int(lay.group_row[e, s]) + i * tb)
                de.append(s)
                rc.append(int(lay.recv_off[s, e]) + i * tb)
                va.append(min(tb, c - i * tb))
    n_remote = len(ex)
    for e in range(E_l):
        c = int(lay.counts[e, r_self])
        for i in range(_ceil_div(c, tb)):
            ex.append(e)
            r0.append(int(lay.group_row[e, r_self]) + i * tb)
            de.append(r_self)
            rc.append(-1)
            va.append(min(tb, c - i * tb))
    a = lambda v: np.array(v, dtype=np.int64)
    return Bands(a(ex), a(r0), a(de), a(rc), a(va), n_remote)


@dataclasses.dataclass
class Segments:
    band0: np.ndarray     # index (in schedule order) of the first band of the segment
    nbands: np.ndarray
    dest: np.ndarray
    src_row: np.ndarray   # first row in the packed output
    dst_row: np.ndarray   # first row in dest's receive buffer
    rows: np.ndarray      # valid rows moved by the one contiguous write


def segments(b: Bands, mgb: int) -> Segments:
    """Transfer segments of [TLS] sec. 3.3.2 and Figure 3(b): a segment is one
    or more consecutive row bands; the first and the last segment hold one band;
    the middle ones hold x = mgb bands (the last middle one may hold fewer).

    Reading: the first/last rule applies per (expert, destination) group,
    because one contiguous single-destination write cannot span two groups.
    """
    out = {k: [] for k in ("band0", "nbands", "dest", "src_row", "dst_row", "rows")}
    i = 0
    n = b.n_remote
    while i < n:
        j = i
        while j < n and b.expert[j] == b.expert[i] and b.dest[j] == b.dest[i]:
            j += 1
        nb = j - i
        sizes = [1] if nb == 1 else ([1, 1] if nb == 2 else None)
        if sizes is None:
            mid = nb - 2
            sizes = [1] + [min(mgb, mid - q) for q in range(0, mid, mgb)] + [1]
        p = i
        for sz in sizes:
            out["band0"].append(p)
            out["nbands"].append(sz)
            out["dest"].append(int(b.dest[p]))
            out["src_row"].append(int(b.row0[p]))
            out["dst_row"].append(int(b.recv0[p]))
            out["rows"].append(int(sum(b.valid[p:p + sz])))
            p += sz
        i = j
    return Segments(**{k: np.array(v, dtype=np.int64) for k, v in out.items()})


# --------------------------------------------------------------------------
# step 5: expert FFN  ([TLS] sec. 2.1 step 3; FFN form as specified for the path)
# --------------------------------------------------------------------------

def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def expert_ffn(X: np.ndarray, W1: np.ndarray, W3: Optional[np.ndarray], W2: np.ndarray) -> np.ndarray:
    """One expert's FFN on its rows, fp64.

    gated:     Y = (SiLU(X W1^T) * (X W3^T)) W2^T
    non-gated: Y = SiLU(X W1^T) W2^T
    W1, W3 are [F, H] and W2 is [H, F] (out x in), given as float64.
    """
    u = X @ W1.T
    h = silu(u) * (X @ W3.T) if W3 is not None else silu(u)
    return h @ W2.T


def expert_outputs(x_perm: np.ndarray, lay: Layout, W1b, W3b, W2b) -> np.ndarray:
    """y_perm: every expert's FFN applied to its rows X_e; zero rows stay zero.

    [TLS] sec. 3.2: each expert keeps its own A, B and C; padding rows take
    part in the GEMM (and come out as zero rows since FFN(0) = 0 here).
    """
    y = np.zeros((lay.m_pad, W2b.shape[1]), dtype=np.float64)
    for e in range(lay.E_l):
        lo, n = int(lay.expert_base[e]), int(lay.M_e[e])
        if n == 0:
            continue
        W3 = widen_bf16(W3b[e]) if W3b is not None else None
        y[lo:lo + n] = expert_ffn(x_perm[lo:lo + n], widen_bf16(W1b[e]), W3, widen_bf16(W2b[e]))
    return y


# --------------------------------------------------------------------------
# step 6: the second all-to-all (combine transfer) and weighted reduction
#         ([TLS] sec. 2.1 steps 4-5; sec. 3.2.3)
# --------------------------------------------------------------------------

def combine_transfer(y_perm: np.ndarray, b: Bands, lay: Layout) -> List[Optional[np.ndarray]]:
    """Rank s's receive buffer after the transfer: valid rows of every remote
    band land at the plan's receive offset ([TLS] sec. 3.2.3). None for r_self."""
    H = y_perm.shape[1]
    bufs: List[Optional[np.ndarray]] = []
    for s in range(lay.R):
        bufs.append(None if s == lay.r_self else np.zeros((int(lay.recv_rows[s]), H), dtype=np.float64))
    for i in range(b.n_remote):
        s, n = int(b.dest[i]), int(b.valid[i])
        bufs[s][b.recv0[i]:b.recv0[i] + n] = y_perm[b.row0[i]:b.row0[i] + n]
    return bufs


def weighted_reduction(bufs, y_perm: np.ndarray, gates: np.ndarray, lay: Layout) -> np.ndarray:
    """Scale step ([TLS] sec. 2.1 step 5): for every token (s, t),
    y[s, t] = sum over slots j (ascending) whose expert is local to r_self of
    gate[s, t, j] * (the returned row). Tokens with no local slot get 0.
    Returns float64 [R, T, H]: this rank's share of every token's output."""
    R, T = lay.R, lay.T
    H = y_perm.shape[1]
    out = np.zeros((R * T, H), dtype=np.float64)
    for g in range(R * T):
        s = g // T
        for j in range(lay.recv_row.shape[1]):
            r = int(lay.recv_row[g, j])
            if r < 0:
                continue
            row = y_perm[r] if s == lay.r_self else bufs[s][r]
            out[g] += gates[g, j] * row
    return out.reshape(R, T, H)


# --------------------------------------------------------------------------
# the whole share
# --------------------------------------------------------------------------

@dataclasses.dataclass
class ShareResult:
    ids: np.ndarray
    gates: np.ndarray
    layout: Layout
    bands: Bands
    segs: Segments
    x_perm: np.ndarray
    y_perm: np.ndarray
    bufs: list
    y_share: np.ndarray


def oracle_share(logits, x_bits, W1b, W3b, W2b, *, R: int, T: int, E: int, k: int,
                 gate_kind: str, r_self: int, tb_m: int, mgb: int = 1,
                 with_ffn: bool = True, with_rows: bool = True) -> ShareResult:
    """Route -> layout -> schedule/plan -> per-expert FFN -> transfer -> reduction.

    [TLS] sec. 2.1 (the five steps of a distributed MoE forward, with the
    dispatch modelled as a gather of this rank's rows) and sec. 3.2-3.3.
    W1b/W3b/W2b hold rank r_self's local experts only (bf16 bits).
    with_ffn False stops after the plan and the gathered rows; with_rows
    False (only without the FFN) also leaves out the gathered rows (x_perm
    None), for shapes whose float64 rows would not fit in memory.
    """
    E_l = E // R
    ids, gates = route(logits, k, gate_kind)
    lay = row_layout(ids, R, T, E_l, r_self, tb_m)
    b = tile_schedule(lay)
    sg = segments(b, mgb)
    x_perm = gather_rows(x_bits, lay) if (with_ffn or with_rows) else None
    if not with_ffn:
        return ShareResult(ids, gates, lay, b, sg, x_perm, None, None, None)
    y_perm = expert_outputs(x_perm, lay, W1b, W3b, W2b)
    bufs = combine_transfer(y_perm, b, lay)
    y = weighted_reduction(bufs, y_perm, gates, lay)
    return ShareResult(ids, gates, lay, b, sg, x_perm, y_perm, bufs, y)


def token_rows(res: ShareResult, W1b, W3b, W2b, tokens, x_bits=None) -> np.ndarray:
    """y_share rows of selected tokens only, from the definition
    y[g] = sum_j gate_j * FFN_{e_j}(x_g) over the local slots of g (for sampled
    checks where the full share is too slow). Works one expert at a time so
    only one expert's weights are widened to float64 at once. x_g comes from
    the gathered rows, or from x_bits [R, T, H] when the result holds none.
    tokens: global token indices. Returns float64 [len, H]."""
    lay = res.layout
    H = W2b.shape[1]
    first = lay.r_self * lay.E_l
    tokens = [int(g) for g in tokens]
    out = np.zeros((len(tokens), H), dtype=np.float64)
    xrow = {}
    for q, g in enumerate(tokens):
        hit = np.nonzero(lay.row_src == g)[0]
        if hit.size:
            xrow[g] = (res.x_perm[hit[0]] if res.x_perm is not None
                       else widen_bf16(x_bits.reshape(-1, x_bits.shape[-1])[g]))
    for e in range(lay.E_l):
        pairs = [(q, j) for q, g in enumerate(tokens) for j in range(res.ids.shape[1])
                 if int(res.ids[g, j]) - first == e]
        if not pairs:
            continue
        X = np.stack([xrow[tokens[q]] for q, _ in pairs])
        W3 = widen_bf16(W3b[e]) if W3b is not None else None
        Y = expert_ffn(X, widen_bf16(W1b[e]), W3, widen_bf16(W2b[e]))
        for (q, j), y in zip(pairs, Y):
            out[q] += res.gates[tokens[q], j] * y
    return out
