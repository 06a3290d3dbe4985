// Expert problem construction of the tile-signalling overlap paper
// (sec. 3.2): the remote-owner-aligned row layout (sec. 3.2.1, Algorithm 1),
// the remote-first row-band schedule (sec. 3.2.2), the combine plan
// (sec. 3.2.3) and the transfer segments (sec. 3.3.2, Fig. 3(b)); then the
// gather of every routed row into its packed position (the dispatch,
// modelled on one GPU) and the zero fill of the padding rows.
//
// Layout: for each local expert, owner groups in ascending remote rank, the
// local rank last; a remote group is padded with zero rows to a multiple of
// tb_m; rows inside a group follow the owner's token order. Experts sit in
// one buffer at tb_m-aligned bases. Band schedule: experts ordered by
// (remote band count desc, remote rows desc, id asc), their remote bands in
// layout order, then all local bands by expert id. Segments per (expert,
// destination) group: 1 band, middle segments of mgb bands, 1 band.
//
// GEMM row tiles (independent of the band height): expert e's tb_m-aligned
// rows are cut into tiles of kTileM rows from its base (the last one shorter).
// GEMM schedule: every tile that holds a remote band, experts in the band
// schedule's order, then the remaining tiles by expert id. A segment's rows
// lie in one expert, so the tiles covering it are consecutive.
//
// With the gather fused into the first projection's tile loads the rows are
// not copied: only the indexes are built (row_src, -1 for padding). The plan
// also zeroes the one row of H zeros that padding rows read there when x is
// too large for the buffer-resource loads (2 GiB or more).
#include "common.hpp"
#include "partition_model.hpp"

namespace moe {

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int nseg_of(int nb, int mgb) {
  return nb <= 2 ? nb : 2 + ceil_div(nb - 2, mgb);
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxEl = 256;
constexpr int kPlanMaxGroups = 2048;  // E_l * R limit (checked on the host)

// device evaluation of the CU-split model: bounds of its LDS tables (past
// them the choice falls back to calib.c_min, with META_PRED = -1)
constexpr int kPartPos = 2048;     // row tiles
constexpr int kPartSegs = 2048;    // segments
constexpr int kPartWaves = 2048;   // producer waves over all candidates
constexpr int kPartCand = 64;      // candidates

// In-place exclusive scan of a[0, n) in LDS by the whole workgroup
// (kPlanThreads threads, any n: each thread scans a run of ceil(n / threads)
// elements); returns the total. s_w: 17 ints of scratch.
__device__ int block_exscan(int* a, int n, int* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += a[i];
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) { const int v = s_w[w]; s_w[w] = acc; acc += v; }
    s_w[16] = acc;
  }
  __syncthreads();
  int run = s_w[wave] + incl - local;
  for (int i = lo; i < hi; ++i) { const int v = a[i]; a[i] = run; run += v; }
  const int total = s_w[16];
  __syncthreads();
  return total;
}

// largest k < n with a[k] <= v (a ascending, a[0] <= v): the run holding v
__device__ __forceinline__ int find_run(const int* a, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Single workgroup; every phase is parallel over experts, groups, bands,
// segments or tiles, and every offset is an exclusive scan.
//  * groups (e, s) are indexed e * R + s (layout order inside an expert:
//    remote owners ascending, then the local owner);
//  * remote groups in schedule order are k = o (R - 1) + q: expert order[o]
//    (rule (ii)), the q-th remote owner;
//  * bands: the remote groups' bands in schedule order, then the local
//    bands by expert id (rule (i)); segments: per remote group 1, mgb, ...,
//    mgb, (remainder), 1 bands.
__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ counts, moe_plan_t p,
                                                        u32x4* __restrict__ zero_row, const moe_calib_t calib,
                                                        int R, int El, int r_self, int tb, int mgb, int H,
                                                        int F) {
  __shared__ int s_cnt[kPlanMaxGroups];
  __shared__ int s_rel[kPlanMaxGroups];            // group start relative to its expert base
  __shared__ int s_goff[2 * kPlanMaxGroups + 1];   // remote groups (schedule order): bands | segments
  __shared__ int s_eoff[5 * kPlanMaxEl + 1];       // per expert: rows | tiles | local bands | remote tiles | other tiles
  __shared__ int s_alg[kPlanMaxEl];                // tb-aligned rows of expert e
  __shared__ int s_nrb[kPlanMaxEl], s_nrr[kPlanMaxEl], s_rank[kPlanMaxEl], s_order[kPlanMaxEl];
  __shared__ int s_trpos[kPlanMaxEl];              // schedule position of e's first remote tile
  __shared__ int s_w[17];
  __shared__ double s_tt[kPartPos];      // model: instance time of the row tile at each position
  __shared__ double s_wv[kPartWaves];    // model: wave lengths, then wave ends, per candidate
  __shared__ int s_spos[kPartSegs];      // model: position of each segment's last row tile
  __shared__ int s_sfrom[kPartSegs];     // model: valid rows of segments i, i+1, ...
  __shared__ int s_woff[kPartCand + 1];  // model: first wave of each candidate
  __shared__ double s_tprod[kPartCand];
  __shared__ double s_total[kPartCand];
  __shared__ int s_fit;
  const int tid = threadIdx.x;
  const int G = El * R, Rr = R - 1, K = El * Rr;
  const int tsh = __ffs(tb) - 1;   // tb is a power of two
  for (int i = tid; i < H / 8; i += kPlanThreads) zero_row[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < kCtrWords; i += kPlanThreads) p.tile_ctr[i] = 0;
  for (int i = tid; i < G; i += kPlanThreads) s_cnt[i] = counts[i];
  for (int e = tid; e < El; e += kPlanThreads) s_rank[e] = 0;
  __syncthreads();

  // per expert: group starts, aligned rows, remote bands / rows
  for (int e = tid; e < El; e += kPlanThreads) {
    int rel = 0, nrb = 0, nrr = 0;
    for (int q = 0; q < R; ++q) {           // remote owners ascending, then the local owner
      const int s = (q < Rr) ? (q < r_self ? q : q + 1) : r_self;
      const int c = s_cnt[e * R + s];
      s_rel[e * R + s] = rel;
      if (s != r_self) {
        const int nb = (c + tb - 1) >> tsh;
        rel += nb << tsh;
        nrb += nb;
        nrr += c;
      } else {
        rel += c;
      }
    }
    s_alg[e] = ((rel + tb - 1) >> tsh) << tsh;
    s_nrb[e] = nrb;
    s_nrr[e] = nrr;
  }
  // receive offsets: (expert, token) order in each owner's combine buffer
  for (int i = tid; i < G; i += kPlanThreads) {
    const int e = i / R, s = i - (i / R) * R;
    int acc = 0;
    for (int f = 0; f < e; ++f) acc += s_cnt[f * R + s];
    p.recv_off[s * El + e] = acc;
  }
  __syncthreads();
  // rule (ii): rank of expert e under (remote bands desc, remote rows desc, id asc)
  for (int i = tid; i < El * El; i += kPlanThreads) {
    const int e = i / El, f = i - (i / El) * El;
    const bool before = s_nrb[f] > s_nrb[e] ||
                        (s_nrb[f] == s_nrb[e] && (s_nrr[f] > s_nrr[e] || (s_nrr[f] == s_nrr[e] && f < e)));
    if (before) atomicAdd(&s_rank[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < El; e += kPlanThreads) s_order[s_rank[e]] = e;
  __syncthreads();

  // per-expert offsets, one scan over five concatenated runs
  for (int e = tid; e < El; e += kPlanThreads) {
    const int nt = ceil_div(s_alg[e], kTileM), nrt = ceil_div(s_rel[e * R + r_self], kTileM);
    s_eoff[e] = s_alg[e];
    s_eoff[El + e] = nt;
    s_eoff[2 * El + e] = (s_cnt[e * R + r_self] + tb - 1) >> tsh;
    s_eoff[3 * El + s_rank[e]] = nrt;   // remote tiles, experts in rule-(ii) order
    s_eoff[4 * El + e] = nt - nrt;
  }
  // per remote group in schedule order: bands | segments
  for (int k = tid; k < K; k += kPlanThreads) {
    const int o = k / Rr, q = k - (k / Rr) * Rr;
    const int e = s_order[o], s = q < r_self ? q : q + 1;
    const int nb = (s_cnt[e * R + s] + tb - 1) >> tsh;
    s_goff[k] = nb;
    s_goff[K + k] = nseg_of(nb, mgb);
  }
  __syncthreads();
  const int etot = block_exscan(s_eoff, 5 * El, s_w);
  const int gtot = block_exscan(s_goff, 2 * K, s_w);
  const int* e_base = s_eoff;                   // first packed row of expert e
  const int m_pad = s_eoff[El];
  const int* e_tbase = s_eoff + El;             // + m_pad: first row tile (layout id)
  const int n_tiles = s_eoff[2 * El] - m_pad;
  const int* e_loff = s_eoff + 2 * El;          // + s_eoff[2 El]: first local band (after the remote ones)
  const int n_remote_tiles = s_eoff[4 * El] - s_eoff[3 * El];
  const int n_remote = K > 0 ? s_goff[K] : 0;   // remote bands
  const int n_seg = gtot - n_remote;
  const int n_bands = n_remote + (s_eoff[3 * El] - s_eoff[2 * El]);
  (void)etot;
  for (int e = tid; e < El; e += kPlanThreads)
    s_trpos[e] = s_eoff[3 * El + s_rank[e]] - s_eoff[3 * El];
  if (tid == 0) {
    p.meta[META_NRTILES] = n_remote_tiles;
    p.meta[META_NTILES] = n_tiles;
    p.meta[META_MPAD] = m_pad;
    p.meta[META_NBANDS] = n_bands;
    p.meta[META_NREMOTE] = n_remote;
    p.meta[META_NSEG] = n_seg;
    p.meta[META_STATUS] = 0;
  }
  for (int e = tid; e <= El; e += kPlanThreads) p.expert_base[e] = e < El ? e_base[e] : m_pad;
  __syncthreads();

  // one pass: row tiles, groups, bands, segments
  const int n_work = n_tiles + G + n_bands + n_seg;
  for (int i = tid; i < n_work; i += kPlanThreads) {
    if (i < n_tiles) {
      const int t = i;
      const int e = find_run(e_tbase, El, t + m_pad);
      const int j = t + m_pad - e_tbase[e];
      const int nrt = ceil_div(s_rel[e * R + r_self], kTileM);
      p.tile_row0[t] = e_base[e] + j * kTileM;
      p.tile_expert[t] = e;
      p.tile_rows[t] = min(kTileM, s_alg[e] - j * kTileM);
      const int lpos = n_remote_tiles + (s_eoff[4 * El + e] - s_eoff[4 * El]);
      p.tile_sched[j < nrt ? s_trpos[e] + j : lpos + (j - nrt)] = t;
      continue;
    }
    int w = i - n_tiles;
    if (w < G) {
      p.group_row[w] = e_base[w / R] + s_rel[w];
      continue;
    }
    w -= G;
    if (w < n_bands) {
      const int b = w;
      int e, s, j;
      if (b < n_remote) {
        const int k = find_run(s_goff, K, b);
        e = s_order[k / Rr];
        const int q = k - (k / Rr) * Rr;
        s = q < r_self ? q : q + 1;
        j = b - s_goff[k];
      } else {
        const int lb = b - n_remote + e_loff[0];
        e = find_run(e_loff, El, lb);
        s = r_self;
        j = lb - e_loff[e];
      }
      const int c = s_cnt[e * R + s];
      const int row0 = e_base[e] + s_rel[e * R + s] + (j << tsh);
      const int valid = min(tb, c - (j << tsh));
      p.band_row0[b] = row0;
      p.band_expert[b] = e;
      p.band_dest[b] = s;
      p.band_recv0[b] = (s != r_self) ? p.recv_off[s * El + e] + (j << tsh) : -1;
      p.band_valid[b] = valid;
      p.slot_valid[row0 >> tsh] = valid;
      continue;
    }
    const int sg = w - n_bands;
    const int k = find_run(s_goff + K, K, sg + n_remote);
    const int e = s_order[k / Rr];
    const int q = k - (k / Rr) * Rr;
    const int s = q < r_self ? q : q + 1;
    const int c = s_cnt[e * R + s];
    const int nb = (c + tb - 1) >> tsh;
    const int ns = nseg_of(nb, mgb);
    const int qi = sg + n_remote - s_goff[K + k];   // segment index inside the group
    const int j = qi == 0 ? 0 : (qi == ns - 1 ? nb - 1 : 1 + (qi - 1) * mgb);
    const int sz = (qi == 0 || qi == ns - 1) ? 1 : min(mgb, nb - 1 - j);
    const int grow = e_base[e] + s_rel[e * R + s];   // the group's first packed row
    p.seg_band0[sg] = s_goff[k] + j;
    p.seg_nbands[sg] = sz;
    p.seg_dest[sg] = s;
    p.seg_src_row[sg] = grow + (j << tsh);
    p.seg_dst_row[sg] = p.recv_off[s * El + e] + (j << tsh);
    p.seg_rows[sg] = min(c - (j << tsh), sz << tsh);
    p.seg_tile0[sg] = (e_tbase[e] - m_pad) + (s_rel[e * R + s] + (j << tsh)) / kTileM;
    p.seg_tile1[sg] = (e_tbase[e] - m_pad) + (s_rel[e * R + s] + ((j + sz) << tsh) - 1) / kTileM;
  }
  __syncthreads();

  // copy units: exclusive prefix of ceil(segment bytes / kCopyUnitBytes)
  const int per = (n_seg + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n_seg, tid * per), hi = min(n_seg, lo + per);
  const int lane = tid & 63, wave = tid >> 6;
  auto units = [&](int sg) {
    return (int)(((long)p.seg_rows[sg] * H * 2 + kCopyUnitBytes - 1) / kCopyUnitBytes);
  };
  {
    int local = 0;
    for (int sg = lo; sg < hi; ++sg) local += units(sg);
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int w = 0; w < kPlanThreads / 64; ++w) { const int v = s_w[w]; s_w[w] = acc; acc += v; }
      p.meta[META_NUNITS] = acc;
    }
    __syncthreads();
    int acc = s_w[wave] + incl - local;
    for (int sg = lo; sg < hi; ++sg) { p.seg_unit0[sg] = acc; acc += units(sg); }
  }

  // ---- the CU-split model (partition_model.hpp) for this plan's row tiles
  // and segments, the same closed form as moe_plan_partition
  const int n_pos = n_tiles;
  const int tiles2 = (H + kModelTileCols - 1) / kModelTileCols;
  const int n_cand = (calib.c_max - calib.c_min) / calib.c_step + 1;
  __syncthreads();   // s_w is reused below
  if (tid == 0) {
    int fit = n_pos <= kPartPos && n_seg <= kPartSegs && n_cand >= 1 && n_cand <= kPartCand;
    int w = 0;
    for (int ci = 0; fit && ci < n_cand; ++ci) {
      const long P = calib.n_cu - (calib.c_min + ci * calib.c_step);
      s_woff[ci] = w;
      w += (int)(((long)n_pos * tiles2 + P - 1) / P);
      if (w > kPartWaves) fit = 0;
    }
    if (fit) s_woff[n_cand] = w;
    s_fit = fit;
  }
  __syncthreads();
  if (!s_fit) {
    if (tid == 0) {
      p.meta[META_CAUTO] = calib.c_min;
      *reinterpret_cast<double*>(p.meta + META_PRED) = -1.0;
    }
    return;
  }
  for (int q = tid; q < n_pos; q += kPlanThreads) {   // instance time per schedule position
    const int rt = p.tile_sched[q];
    const int e = p.tile_expert[rt];
    const long m_e = (long)s_rel[e * R + r_self] + s_cnt[e * R + r_self];   // the local group is last
    s_tt[q] = model_tile_time(p.tile_rows[rt], F, model_rate(calib, m_e));
  }
  // segments: position of the last row tile (remote tiles of expert e sit at
  // positions s_trpos[e] + j) and the valid rows from each segment on
  // (integers: the total minus an exclusive prefix)
  for (int sg = tid; sg < n_seg; sg += kPlanThreads) {
    const int e = p.band_expert[p.seg_band0[sg]];
    s_spos[sg] = s_trpos[e] + (p.seg_tile1[sg] - (e_tbase[e] - m_pad));
    s_sfrom[sg] = p.seg_rows[sg];
  }
  __syncthreads();
  const int rtot = block_exscan(s_sfrom, n_seg, s_w);
  for (int sg = tid; sg < n_seg; sg += kPlanThreads) s_sfrom[sg] = rtot - s_sfrom[sg];
  // producer waves: lengths (maxima over the positions each wave covers)
  const int tw = s_woff[n_cand];
  for (int idx = tid; idx < tw; idx += kPlanThreads) {
    int ci = 0;
    while (s_woff[ci + 1] <= idx) ++ci;
    const long P = calib.n_cu - (calib.c_min + ci * calib.c_step);
    long p0, p1;
    model_wave_span(idx - s_woff[ci], P, tiles2, n_pos, &p0, &p1);
    double len = 0.0;
    for (long q = p0; q <= p1; ++q) len = len > s_tt[q] ? len : s_tt[q];
    s_wv[idx] = len;
  }
  __syncthreads();
  if (tid < n_cand) {   // wave ends, in order
    const long P = calib.n_cu - (calib.c_min + tid * calib.c_step);
    const long n_inst = (long)n_pos * tiles2;
    double t = 0.0;
    for (int w = s_woff[tid]; w < s_woff[tid + 1]; ++w) {
      const long wi = w - s_woff[tid];
      t = model_wave_end(t, s_wv[w], n_inst - wi * P < P ? n_inst - wi * P : P, P);
      s_wv[w] = t;
    }
    s_tprod[tid] = t;
  }
  __syncthreads();
  // copy end per candidate: one wave each
  for (int ci = wave; ci < n_cand; ci += kPlanThreads / 64) {
    const int c = calib.c_min + ci * calib.c_step;
    const long P = calib.n_cu - c;
    const double bw = model_copy_bw(calib, c);
    double tc = 0.0;
    for (int sg = lane; sg < n_seg; sg += 64) {
      const double r = s_wv[s_woff[ci] + (int)(((long)s_spos[sg] * tiles2 + tiles2 - 1) / P)];
      const double v = model_copy_end(r, s_sfrom[sg], H, bw);
      tc = tc > v ? tc : v;
    }
    for (int d = 32; d > 0; d >>= 1) {
      const double o = __shfl_xor(tc, d, 64);
      tc = tc > o ? tc : o;
    }
    if (lane == 0) s_total[ci] = model_total(s_tprod[ci], tc, n_seg > 0, calib.seg_latency_s);
  }
  __syncthreads();
  if (tid == 0) {
    double best_t = 0.0;
    int best_c = -1;
    for (int ci = 0; ci < n_cand; ++ci)
      if (best_c < 0 || s_total[ci] < best_t) { best_t = s_total[ci]; best_c = calib.c_min + ci * calib.c_step; }
    p.meta[META_CAUTO] = best_c;
    *reinterpret_cast<double*>(p.meta + META_PRED) = best_t;
  }
}

// index: every local (token, slot) -> its packed row; writes row_src and recv_row.
// One block per routing chunk (<= 256 tokens of one source rank); thread = token.
// Rank inside the (expert, owner) group = rows of earlier chunks + rows of
// earlier waves of this chunk + earlier lanes of this wave. Each (token, slot)
// sets its lane's bit in an LDS bitmap of expert e and its wave (tokens hold
// distinct experts), so a rank is one popcount; the chunk's group bases sit
// in LDS. The blocks also mark every padding row of [0, m_pad) (row_src = -1;
// a row is padding unless it is one of the valid rows of its band slot),
// rows grid-stride: disjoint from the rows the tokens fill.
__global__ __launch_bounds__(256) void k_gather_index(const int32_t* __restrict__ ids, moe_plan_t p,
                                                       int R, int T, int k, int El, int first_local,
                                                       int r_self, int chunks_per_rank, int tb) {
  __shared__ unsigned long long s_bits[kPlanMaxEl][4];   // tokens of this chunk per (expert, wave)
  __shared__ int s_wbase[kPlanMaxEl][4];                 // rows before (expert, wave) in the group
  __shared__ int s_gr[kPlanMaxEl];   // first packed row of group (e, s)
  __shared__ int s_ro[kPlanMaxEl];   // first combine-buffer row of group (e, s)
  const int chunk = blockIdx.x;
  const int s = chunk / chunks_per_rank;
  const int t0 = (chunk % chunks_per_rank) * kChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = t0 + tid;
  const bool active = t < T;
  const int g = s * T + (active ? t : 0);
  for (int i = tid; i < El * 4; i += blockDim.x) s_bits[i >> 2][i & 3] = 0ull;
  for (int e = tid; e < El; e += blockDim.x) {
    s_wbase[e][0] = p.chunk_base[chunk * El + e];
    s_gr[e] = p.group_row[e * R + s];
    s_ro[e] = p.recv_off[s * El + e];
  }
  // unconditional loads with clamped indices (predicated ones would each wait
  // for the previous), then the selection
  int my[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) my[j] = ids[g * k + (j < k ? j : k - 1)] - first_local;
#pragma unroll
  for (int j = 0; j < 16; ++j) my[j] = (active && j < k && my[j] >= 0 && my[j] < El) ? my[j] : -1;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (my[j] >= 0) atomicOr(&s_bits[my[j]][wave], 1ull << lane);
  __syncthreads();
  for (int e = tid; e < El; e += blockDim.x) {   // prefix over the 4 waves
    int acc = s_wbase[e][0];
    for (int w = 0; w < 4; ++w) { s_wbase[e][w] = acc; acc += __popcll(s_bits[e][w]); }
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (!active || j >= k) continue;
    const int e = my[j];
    if (e < 0) {   // expert not local
      p.recv_row[g * k + j] = -1;
      continue;
    }
    const int rank = s_wbase[e][wave] + __popcll(s_bits[e][wave] & lt);
    const int row = s_gr[e] + rank;
    p.row_src[row] = g;
    p.recv_row[g * k + j] = (s == r_self) ? row : s_ro[e] + rank;
  }
  const int m_pad = p.meta[META_MPAD];
  for (int r = blockIdx.x * 256 + tid; r < m_pad; r += gridDim.x * 256)
    if ((r % tb) >= p.slot_valid[r / tb]) p.row_src[r] = -1;
}

// copy: row r of [0, m_pad) gets x of token row_src[r] when it is one of the
// valid rows of its band slot, else zeros (owner-boundary padding, or the
// aligned gap after an expert). One wave per row, 16-byte vectors,
// grid-stride over rows.
__global__ __launch_bounds__(256) void k_gather_copy(const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ x_perm, moe_plan_t p,
                                                      int H, int tb) {
  const int m_pad = p.meta[META_MPAD];
  const int lane = threadIdx.x & 63;
  const int nv = H / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < m_pad; r += gridDim.x * 4) {
    u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (size_t)r * H);
    if ((r % tb) < p.slot_valid[r / tb]) {
      const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)p.row_src[r] * H);
      int v = lane;
      for (; v + 192 < nv; v += 256) {
        const u32x4 a = src[v], b = src[v + 64], c = src[v + 128], d = src[v + 192];
        dst[v] = a; dst[v + 64] = b; dst[v + 128] = c; dst[v + 192] = d;
      }
      for (; v < nv; v += 64) dst[v] = src[v];
    } else {
      for (int v = lane; v < nv; v += 64) dst[v] = z;
    }
  }
}

hipError_t launch_plan(const Geometry& g, const int32_t* counts, const moe_plan_t& p, uint16_t* zero_row,
                       const moe_calib_t& calib, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, counts, p, reinterpret_cast<u32x4*>(zero_row), calib,
                     g.R, g.El, g.r_self, g.tb_m, g.mgb, g.H, g.F);
  return hipGetLastError();
}

hipError_t launch_gather(const Geometry& g, const uint16_t* x, const int32_t* ids,
                         uint16_t* x_perm, const moe_plan_t& p, hipStream_t st) {
  hipLaunchKernelGGL(k_gather_index, dim3(g.n_chunks), dim3(256), 0, st, ids, p, g.R, g.T, g.k, g.El,
                     g.r_self * g.El, g.r_self, g.chunks_per_rank, g.tb_m);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  // grid-stride over at most m_pad_max rows, four rows per block
  const int64_t blocks = (g.m_pad_max + 3) / 4;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_gather_copy, dim3(grid), dim3(256), 0, st, x, x_perm, p, g.H, g.tb_m);
  return hipGetLastError();
}

}  // namespace moe
