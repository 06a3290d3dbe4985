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
// also zeroes the one row of H zeros that padding rows read there.
#include "common.hpp"
#include "partition_model.hpp"

namespace moe {

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int nseg_of(int nb, int mgb) {
  return nb <= 2 ? nb : 2 + ceil_div(nb - 2, mgb);
}

constexpr int kPlanMaxEl = 256;
constexpr int kPlanMaxGroups = 2048;  // E_l * R limit (checked on the host)

// device evaluation of the CU-split model: bounds of its LDS tables (past
// them the choice falls back to calib.c_min, with META_PRED = -1)
constexpr int kPartPos = 2048;     // row tiles
constexpr int kPartSegs = 2048;    // segments
constexpr int kPartWaves = 2048;   // producer waves over all candidates
constexpr int kPartCand = 64;      // candidates

// single workgroup: everything here is O(E_l * R) metadata

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ counts, moe_plan_t p,
                                                u32x4* __restrict__ zero_row, const moe_calib_t calib,
                                                int R, int El, int r_self, int tb, int mgb, int H, int F) {
  __shared__ int s_cnt[kPlanMaxGroups];
  __shared__ int s_rel[kPlanMaxGroups];      // group start relative to its expert base
  __shared__ int s_bandoff[kPlanMaxGroups];  // first band index of the group (schedule order)
  __shared__ int s_segoff[kPlanMaxGroups];   // first segment index (remote groups)
  __shared__ int s_base[kPlanMaxEl + 1];
  __shared__ int s_alg[kPlanMaxEl];          // tb-aligned rows of expert e
  __shared__ int s_nrb[kPlanMaxEl], s_nrr[kPlanMaxEl], s_nlb[kPlanMaxEl], s_order[kPlanMaxEl];
  __shared__ int s_nseg;
  __shared__ int s_tbase[kPlanMaxEl + 1];   // first row tile of expert e
  __shared__ int s_trpos[kPlanMaxEl];       // schedule position of e's first remote tile
  __shared__ int s_tlpos[kPlanMaxEl];       // schedule position of e's first local-only tile
  __shared__ int s_usum[16];             // per-wave totals of the copy-unit scan
  __shared__ double s_tt[kPartPos];      // model: instance time of the row tile at each position
  __shared__ double s_wv[kPartWaves];    // model: wave lengths, then wave ends, per candidate
  __shared__ int s_spos[kPartSegs];      // model: position of each segment's last row tile
  __shared__ int s_sfrom[kPartSegs];     // model: valid rows of segments i, i+1, ...
  __shared__ int s_woff[kPartCand + 1];  // model: first wave of each candidate
  __shared__ double s_tprod[kPartCand];
  __shared__ double s_red[16];
  __shared__ int s_fit, s_rtot;
  const int tid = threadIdx.x;
  const int G = El * R;
  for (int i = tid; i < H / 8; i += blockDim.x) zero_row[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < G; i += blockDim.x) s_cnt[i] = counts[i];
  __syncthreads();

  for (int e = tid; e < El; e += blockDim.x) {
    int rel = 0, nrb = 0, nrr = 0;
    for (int q = 0; q < R; ++q) {           // remote owners ascending, then the local owner
      const int s = (q < R - 1) ? (q < r_self ? q : q + 1) : r_self;
      const int c = s_cnt[e * R + s];
      s_rel[e * R + s] = rel;
      if (s != r_self) {
        const int nb = ceil_div(c, tb);
        rel += nb * tb;
        nrb += nb;
        nrr += c;
      } else {
        rel += c;
      }
    }
    s_alg[e] = ceil_div(rel, tb) * tb;
    s_nrb[e] = nrb;
    s_nrr[e] = nrr;
    s_nlb[e] = ceil_div(s_cnt[e * R + r_self], tb);
  }
  __syncthreads();
  // rule (ii): rank of expert e under (remote bands desc, remote rows desc, id asc)
  for (int e = tid; e < El; e += blockDim.x) {
    int rank = 0;
    for (int f = 0; f < El; ++f) {
      const bool before = s_nrb[f] > s_nrb[e] ||
                          (s_nrb[f] == s_nrb[e] && (s_nrr[f] > s_nrr[e] ||
                                                    (s_nrr[f] == s_nrr[e] && f < e)));
      rank += before ? 1 : 0;
    }
    s_order[rank] = e;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < El; ++e) { s_base[e] = acc; acc += s_alg[e]; }
    s_base[El] = acc;
    // remote bands: experts in rule-(ii) order, groups in layout order
    int band = 0, seg = 0;
    for (int o = 0; o < El; ++o) {
      const int e = s_order[o];
      for (int q = 0; q < R - 1; ++q) {
        const int s = q < r_self ? q : q + 1;
        const int nb = ceil_div(s_cnt[e * R + s], tb);
        s_bandoff[e * R + s] = band;
        s_segoff[e * R + s] = seg;
        band += nb;
        seg += nseg_of(nb, mgb);
      }
    }
    const int n_remote = band;
    for (int e = 0; e < El; ++e) {             // rule (i): local bands last, by expert id
      s_bandoff[e * R + r_self] = band;
      s_segoff[e * R + r_self] = -1;
      band += s_nlb[e];
    }
    // GEMM row tiles: layout ids, then schedule positions
    int nt = 0;
    for (int e = 0; e < El; ++e) { s_tbase[e] = nt; nt += ceil_div(s_alg[e], kTileM); }
    s_tbase[El] = nt;
    int pos = 0;
    for (int o = 0; o < El; ++o) {
      const int e = s_order[o];
      s_trpos[e] = pos;
      pos += ceil_div(s_rel[e * R + r_self], kTileM);   // tiles reaching into the remote groups
    }
    p.meta[META_NRTILES] = pos;
    for (int e = 0; e < El; ++e) {
      s_tlpos[e] = pos;
      pos += ceil_div(s_alg[e], kTileM) - ceil_div(s_rel[e * R + r_self], kTileM);
    }
    p.meta[META_NTILES] = nt;
    p.meta[META_MPAD] = acc;
    p.meta[META_NBANDS] = band;
    p.meta[META_NREMOTE] = n_remote;
    p.meta[META_NSEG] = seg;
    p.meta[META_STATUS] = 0;
    s_nseg = seg;
  }
  __syncthreads();
  for (int i = tid; i < kCtrWords; i += blockDim.x) p.tile_ctr[i] = 0;
  for (int e = tid; e <= El; e += blockDim.x) p.expert_base[e] = s_base[e];
  for (int e = tid; e < El; e += blockDim.x) {
    const int nt = ceil_div(s_alg[e], kTileM), nrt = ceil_div(s_rel[e * R + r_self], kTileM);
    for (int j = 0; j < nt; ++j) {
      const int t = s_tbase[e] + j;
      p.tile_row0[t] = s_base[e] + j * kTileM;
      p.tile_expert[t] = e;
      p.tile_rows[t] = min(kTileM, s_alg[e] - j * kTileM);
      p.tile_sched[j < nrt ? s_trpos[e] + j : s_tlpos[e] + (j - nrt)] = t;
    }
  }
  for (int s = tid; s < R; s += blockDim.x) {   // receive offsets: (expert, token) order
    int acc = 0;
    for (int e = 0; e < El; ++e) { p.recv_off[s * El + e] = acc; acc += s_cnt[e * R + s]; }
  }
  for (int i = tid; i < G; i += blockDim.x) {
    const int e = i / R, s = i % R;
    const int c = s_cnt[i];
    const int row0 = s_base[e] + s_rel[i];
    p.group_row[i] = row0;
    const int nb = ceil_div(c, tb);
    const int b0 = s_bandoff[i];
    int recv0 = 0;
    if (s != r_self) {
      for (int f = 0; f < e; ++f) recv0 += s_cnt[f * R + s];
    }
    for (int j = 0; j < nb; ++j) {
      const int b = b0 + j;
      p.band_row0[b] = row0 + j * tb;
      p.band_expert[b] = e;
      p.band_dest[b] = s;
      p.band_recv0[b] = (s != r_self) ? recv0 + j * tb : -1;
      p.band_valid[b] = min(tb, c - j * tb);
      p.slot_valid[(row0 + j * tb) / tb] = min(tb, c - j * tb);
    }
    if (s != r_self && nb > 0) {
      int sidx = s_segoff[i];
      int j = 0;
      const int ns = nseg_of(nb, mgb);
      for (int q = 0; q < ns; ++q) {
        int sz;
        if (q == 0 || q == ns - 1) sz = 1;
        else sz = min(mgb, nb - 1 - j);
        const int rows = min(c - j * tb, sz * tb);
        p.seg_band0[sidx] = b0 + j;
        p.seg_nbands[sidx] = sz;
        p.seg_dest[sidx] = s;
        p.seg_src_row[sidx] = row0 + j * tb;
        p.seg_dst_row[sidx] = recv0 + j * tb;
        p.seg_rows[sidx] = rows;
        p.seg_tile0[sidx] = s_tbase[e] + (row0 + j * tb - s_base[e]) / kTileM;
        p.seg_tile1[sidx] = s_tbase[e] + (row0 + (j + sz) * tb - 1 - s_base[e]) / kTileM;
        ++sidx;
        j += sz;
      }
    }
  }
  // copy units: exclusive prefix of ceil(segment bytes / kCopyUnitBytes)
  __syncthreads();
  const int n_seg = s_nseg;
  const int per = (n_seg + (int)blockDim.x - 1) / (int)blockDim.x;
  const int lo = tid * per, hi = min(n_seg, lo + per);
  auto units = [&](int sg) {
    return (int)(((long)p.seg_rows[sg] * H * 2 + kCopyUnitBytes - 1) / kCopyUnitBytes);
  };
  int local = 0;
  for (int sg = lo; sg < hi; ++sg) local += units(sg);
  // exclusive scan over the workgroup: inclusive scan inside each wave, then
  // the waves' totals
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_usum[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < (int)blockDim.x / 64; ++w) { const int v = s_usum[w]; s_usum[w] = acc; acc += v; }
    p.meta[META_NUNITS] = acc;
  }
  __syncthreads();
  int acc = s_usum[wave] + incl - local;
  for (int sg = lo; sg < hi; ++sg) { p.seg_unit0[sg] = acc; acc += units(sg); }

  // ---- the CU-split model (partition_model.hpp) for this plan's row tiles
  // and segments, the same closed form as moe_plan_partition
  const int n_pos = s_tbase[El];
  const int tiles2 = (H + kModelTileCols - 1) / kModelTileCols;
  const int n_cand = (calib.c_max - calib.c_min) / calib.c_step + 1;
  __syncthreads();   // s_usum is reused below
  if (tid == 0) {
    int fit = n_pos <= kPartPos && n_seg <= kPartSegs && n_cand <= kPartCand;
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
  for (int q = tid; q < n_pos; q += blockDim.x) {   // instance time per schedule position
    const int rt = p.tile_sched[q];
    const int e = p.tile_expert[rt];
    const long m_e = (long)s_rel[e * R + r_self] + s_cnt[e * R + r_self];   // the local group is last
    s_tt[q] = model_tile_time(p.tile_rows[rt], F, model_rate(calib, m_e));
  }
  // segments: position of the last row tile (remote tiles of expert e sit at
  // positions s_trpos[e] + j) and the valid rows from each segment on
  // (integers: total minus an exclusive prefix, chunked like the unit scan)
  int rsum = 0;
  for (int sg = lo; sg < hi; ++sg) {
    const int e = p.band_expert[p.seg_band0[sg]];
    s_spos[sg] = s_trpos[e] + (p.seg_tile1[sg] - s_tbase[e]);
    rsum += p.seg_rows[sg];
  }
  int rincl = rsum;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(rincl, d, 64);
    if (lane >= d) rincl += y;
  }
  if (lane == 63) s_usum[wave] = rincl;
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    for (int w = 0; w < (int)blockDim.x / 64; ++w) { const int v = s_usum[w]; s_usum[w] = a; a += v; }
    s_rtot = a;
  }
  __syncthreads();
  int before = s_usum[wave] + rincl - rsum;   // valid rows of the segments before this thread's chunk
  for (int sg = lo; sg < hi; ++sg) { s_sfrom[sg] = s_rtot - before; before += p.seg_rows[sg]; }
  // producer waves: lengths (maxima over the positions each wave covers)
  const int tw = s_woff[n_cand];
  for (int idx = tid; idx < tw; idx += blockDim.x) {
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
  double best_t = 0.0;
  int best_c = -1;
  for (int ci = 0; ci < n_cand; ++ci) {
    const int c = calib.c_min + ci * calib.c_step;
    const long P = calib.n_cu - c;
    const double bw = model_copy_bw(calib, c);
    double tc = 0.0;
    for (int sg = tid; sg < n_seg; sg += blockDim.x) {
      const double r = s_wv[s_woff[ci] + (int)(((long)s_spos[sg] * tiles2 + tiles2 - 1) / P)];
      const double v = model_copy_end(r, s_sfrom[sg], H, bw);
      tc = tc > v ? tc : v;
    }
    for (int d = 32; d > 0; d >>= 1) {
      const double o = __shfl_xor(tc, d, 64);
      tc = tc > o ? tc : o;
    }
    if (lane == 0) s_red[wave] = tc;
    __syncthreads();
    if (tid == 0) {
      double m = 0.0;
      for (int w = 0; w < (int)blockDim.x / 64; ++w) m = m > s_red[w] ? m : s_red[w];
      const double total = model_total(s_tprod[ci], m, n_seg > 0, calib.seg_latency_s);
      if (best_c < 0 || total < best_t) { best_t = total; best_c = c; }
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.meta[META_CAUTO] = best_c;
    *reinterpret_cast<double*>(p.meta + META_PRED) = best_t;
  }
}

// index: every local (token, slot) -> its packed row; writes row_src and recv_row.
// One block per routing chunk (<= 256 tokens of one source rank); thread = token.
// Rank inside the (expert, owner) group = rows of earlier chunks + rows of
// earlier waves of this chunk + earlier lanes of this wave (ballot prefix).
__global__ __launch_bounds__(256) void k_gather_index(const int32_t* __restrict__ ids, moe_plan_t p,
                                                       int R, int T, int k, int El, int first_local,
                                                       int r_self, int chunks_per_rank) {
  __shared__ int s_wcnt[4][kPlanMaxEl];
  const int chunk = blockIdx.x;
  const int s = chunk / chunks_per_rank;
  const int t0 = (chunk % chunks_per_rank) * kChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = t0 + tid;
  const bool active = t < T;
  const int g = s * T + (active ? t : 0);
  int my[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) my[j] = (active && j < k) ? ids[g * k + j] - first_local : -1;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < El; ++e) {
    bool has = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) has |= (my[j] == e);
    const uint64_t m = __ballot(has);
    if (lane == 0) s_wcnt[wave][e] = __popcll(m);
  }
  __syncthreads();
  for (int e = tid; e < El; e += blockDim.x) {   // exclusive prefix over the 4 waves
    int acc = 0;
    for (int w = 0; w < 4; ++w) { const int c = s_wcnt[w][e]; s_wcnt[w][e] = acc; acc += c; }
  }
  __syncthreads();
  for (int e = 0; e < El; ++e) {
    int slot = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j) slot = (my[j] == e) ? j : slot;
    const uint64_t m = __ballot(slot >= 0);
    if (slot >= 0) {
      const int rank = p.chunk_base[chunk * El + e] + s_wcnt[wave][e] + __popcll(m & lt);
      const int row = p.group_row[e * R + s] + rank;
      p.row_src[row] = g;
      p.recv_row[g * k + slot] = (s == r_self) ? row : p.recv_off[s * El + e] + rank;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)   // slots whose expert is not local
    if (active && j < k && (my[j] < 0 || my[j] >= El)) p.recv_row[g * k + j] = -1;
}

// copy: row r of [0, m_pad) gets x of token row_src[r] when it is one of the
// valid rows of its band slot, else zeros (owner-boundary padding, or the
// aligned gap after an expert), and row_src[r] = -1. One wave per row,
// 16-byte vectors, grid-stride over rows.
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
      if (lane == 0) p.row_src[r] = -1;
      for (int v = lane; v < nv; v += 64) dst[v] = z;
    }
  }
}

// index only (the gather fused into the first projection): row_src = -1 for
// every row of [0, m_pad) that is not a valid row of its band slot
__global__ __launch_bounds__(256) void k_pad_index(moe_plan_t p, int tb) {
  const int m_pad = p.meta[META_MPAD];
  for (int r = blockIdx.x * 256 + threadIdx.x; r < m_pad; r += gridDim.x * 256)
    if ((r % tb) >= p.slot_valid[r / tb]) p.row_src[r] = -1;
}

hipError_t launch_plan(const Geometry& g, const int32_t* counts, const moe_plan_t& p, uint16_t* zero_row,
                       const moe_calib_t& calib, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, counts, p, reinterpret_cast<u32x4*>(zero_row), calib,
                     g.R, g.El, g.r_self, g.tb_m, g.mgb, g.H, g.F);
  return hipGetLastError();
}

hipError_t launch_gather(const Geometry& g, const uint16_t* x, const int32_t* ids,
                         uint16_t* x_perm, const moe_plan_t& p, hipStream_t st) {
  hipLaunchKernelGGL(k_gather_index, dim3(g.n_chunks), dim3(256), 0, st, ids, p, g.R, g.T, g.k, g.El,
                     g.r_self * g.El, g.r_self, g.chunks_per_rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (x_perm == nullptr) {
    const int64_t blocks = (g.m_pad_max + 255) / 256;
    hipLaunchKernelGGL(k_pad_index, dim3((int)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, st, p, g.tb_m);
    return hipGetLastError();
  }
  // grid-stride over at most m_pad_max rows, four rows per block
  const int64_t blocks = (g.m_pad_max + 3) / 4;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_gather_copy, dim3(grid), dim3(256), 0, st, x, x_perm, p, g.H, g.tb_m);
  return hipGetLastError();
}

}  // namespace moe
