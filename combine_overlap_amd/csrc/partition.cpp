// Per-layer producer/consumer CU split (pure host function).
//
// The Weave abstract (arXiv 2609.21483) decides the split per layer from the
// routing result so that the communication and computation worker groups
// match the layer's communication/computation throughput ratio; the
// tile-signalling paper (sec. 4.3.4, Fig. 9) shows that too few consumer SMs
// leave a long transfer tail and too many slow the GEMM.
//
// Model (its form is not given on the pages; this is the plainest one that
// uses only the routing counts and measured rates). For c consumer CUs:
//  * the output projection runs on P = n_cu - c CUs; a tile (up to 256 rows
//    of one expert's tb_m-aligned rows x 256 columns, K = F; a short last row
//    tile computes its rows rounded up to 32) takes t_tile = 2 rows 256 F /
//    rate(M_e) on one CU, with rate(M) = gemm_flops_per_cu * M / (M +
//    gemm_m_half) for an expert of M rows; tiles run in waves of P in
//    schedule order (row tiles holding a
//    remote band first, experts by remote band count, then rows, then id; then
//    the other row tiles by expert), so a band is ready when the wave holding
//    the last column tile of its row tile ends; a partial last wave of n tiles
//    lasts max(n / P, 1/3) of a full one (fewer tiles share the memory
//    bandwidth);
//  * the consumer copies the segments in order, each when its bands are ready
//    and the previous copy is done, at BW(c) = c b / (1 + c b / B) with
//    b = copy_bw_per_cu and B = copy_bw_max (linear in c for few CUs,
//    saturating at B: what the copy reaches while the GEMM loads the memory
//    system), plus seg_latency_s once for the last batch;
//  * T(c) = max(producer end, consumer end).
// c = argmin T(c) over c_min, c_min + c_step, ..., <= c_max (smallest c on
// ties). The step defaults to the XCD count: workgroups are dealt to the 8
// XCDs in turn, so a consumer of c = 8j CUs and a producer of 256 - c CUs fill
// every XCD exactly whichever kernel is dispatched first. mgb = 2 when one
// band moves less than half a MiB (transfer bandwidth saturates only at
// MiB-scale transfers, tile-signalling paper Fig. 3(a)), else 1.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "moe_overlap.h"

namespace {

constexpr int kTileRows = 256;   // GEMM row-tile height

struct Band {
  int expert;
  long rel;        // first row relative to the expert's base
  int rows;        // valid rows
  bool group_end;  // last band of its (expert, owner) group
};

}  // namespace

extern "C" int moe_plan_partition(const moe_shape_t* s, const int32_t* counts, const moe_calib_t* calib,
                                  int32_t* n_consumer_cu, int32_t* mgb, double* predicted_s) {
  if (s == nullptr || counts == nullptr || n_consumer_cu == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->R < 1 || s->R > MOE_MAX_RANKS || s->E < 1 || s->E % s->R != 0 || s->r_self < 0 ||
      s->r_self >= s->R || s->H < 1 || s->F < 1 || s->tb_m < 1)
    return MOE_ERR_INVALID_ARG;
  moe_calib_t c0;
  // measured on MI355X over the five synthetic workloads: 3.6-4.4 TFLOP/s per
  // producer CU on the output projection; the consumer moves 121, 208, 309
  // and 407 GB/s with 8, 16, 32 and 48 CUs while the producer runs
  c0.gemm_flops_per_cu = 3.5e12;
  c0.gemm_m_half = 0.0;
  c0.copy_bw_per_cu = 17.8e9;
  c0.copy_bw_max = 800e9;
  c0.seg_latency_s = 10e-6;
  c0.n_cu = 256;
  c0.c_min = 8;
  c0.c_max = 48;
  c0.c_step = 8;
  const moe_calib_t& k = calib ? *calib : c0;
  if (k.n_cu < 2 || k.c_min < 1 || k.c_max < k.c_min || k.c_max >= k.n_cu || k.c_step < 1 ||
      k.gemm_flops_per_cu <= 0 ||
      k.copy_bw_per_cu <= 0 || k.copy_bw_max <= 0 || k.gemm_m_half < 0 || k.seg_latency_s < 0)
    return MOE_ERR_INVALID_ARG;

  const int El = s->E / s->R, R = s->R, tb = s->tb_m, self = s->r_self;
  std::vector<long> m_e(El, 0), rb(El, 0), rr(El, 0);
  for (int e = 0; e < El; ++e)
    for (int q = 0; q < R; ++q) {
      const long c = counts[e * R + q];
      if (c < 0) return MOE_ERR_INVALID_ARG;
      if (q != self) {
        m_e[e] += (c + tb - 1) / tb * tb;
        rb[e] += (c + tb - 1) / tb;
        rr[e] += c;
      } else {
        m_e[e] += c;
      }
    }
  std::vector<int> order(El);
  for (int e = 0; e < El; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    if (rb[a] != rb[b]) return rb[a] > rb[b];
    if (rr[a] != rr[b]) return rr[a] > rr[b];
    return a < b;
  });
  // remote bands in schedule order (the consumer's order)
  std::vector<Band> bands;
  for (int e : order) {
    long rel = 0;
    for (int q = 0; q < R; ++q) {
      if (q == self) continue;
      const long c = counts[e * R + q];
      const long nb = (c + tb - 1) / tb;
      for (long i = 0; i < nb; ++i)
        bands.push_back(Band{e, rel + i * tb, (int)std::min<long>(tb, c - i * tb), i == nb - 1});
      rel += nb * tb;
    }
  }
  const size_t n_remote = bands.size();
  // row tiles in schedule order: those reaching into the remote groups first
  // (experts in band order), then the rest by expert id
  std::vector<int> t_exp, t_idx;
  std::vector<long> t_first(El + 1, 0);
  for (int e = 0; e < El; ++e) {
    const long alg = (m_e[e] + tb - 1) / tb * tb;
    t_first[e + 1] = t_first[e] + (alg + kTileRows - 1) / kTileRows;
  }
  std::vector<long> remote_rows(El, 0);
  for (int e = 0; e < El; ++e) remote_rows[e] = rb[e] * tb;
  for (int e : order)
    for (long j = 0; j < (remote_rows[e] + kTileRows - 1) / kTileRows; ++j) {
      t_exp.push_back(e);
      t_idx.push_back((int)j);
    }
  for (int e = 0; e < El; ++e)
    for (long j = (remote_rows[e] + kTileRows - 1) / kTileRows; j < t_first[e + 1] - t_first[e]; ++j) {
      t_exp.push_back(e);
      t_idx.push_back((int)j);
    }

  const double band_bytes = 2.0 * tb * (double)s->H;
  const int g = band_bytes < 0.5 * 1048576.0 ? 2 : 1;
  const int tiles2 = (s->H + 255) / 256;
  std::vector<double> rate(El);
  for (int e = 0; e < El; ++e) {
    const double m = (double)std::max<long>(m_e[e], 1);
    rate[e] = k.gemm_flops_per_cu * m / (m + k.gemm_m_half);
  }
  auto t_tile = [&](int e, int j) {   // row tile j of expert e
    const long alg = (m_e[e] + tb - 1) / tb * tb;
    const long rows = std::min<long>(kTileRows, alg - (long)j * kTileRows);
    return 2.0 * (double)((rows + 31) / 32 * 32) * 256.0 * (double)s->F / rate[e];
  };
  std::vector<double> tile_done((size_t)t_first[El], 0.0);

  double best_t = INFINITY;
  int best_c = k.c_min;
  std::vector<size_t> pending;
  for (int c = k.c_min; c <= k.c_max; c += k.c_step) {
    const long P = k.n_cu - c;
    // producer: waves of P tiles in schedule order; a wave lasts as long as its slowest tile
    double t = 0.0, wave_len = 0.0;
    long in_wave = 0;
    pending.clear();
    for (size_t r = 0; r < t_exp.size(); ++r) {
      const size_t id = (size_t)(t_first[t_exp[r]] + t_idx[r]);
      for (int j = 0; j < tiles2; ++j) {
        wave_len = std::max(wave_len, t_tile(t_exp[r], t_idx[r]));
        if (++in_wave == P) {
          t += wave_len;
          for (size_t q : pending) tile_done[q] = t;
          pending.clear();
          in_wave = 0;
          wave_len = 0.0;
          if (j == tiles2 - 1) tile_done[id] = t;
        }
      }
      if (in_wave != 0) pending.push_back(id);
    }
    if (in_wave > 0) {
      t += wave_len * std::max((double)in_wave / (double)P, 1.0 / 3.0);
      for (size_t q : pending) tile_done[q] = t;
    }
    const double t_prod = t;
    // consumer: segments of 1, g, ..., g, 1 bands per group, copied in order
    const double bw = c * k.copy_bw_per_cu / (1.0 + c * k.copy_bw_per_cu / k.copy_bw_max);
    double tc = 0.0;
    size_t b = 0;
    while (b < n_remote) {
      size_t last = b;
      while (last < n_remote && !bands[last].group_end) ++last;
      const size_t nb = last - b + 1;
      for (size_t p = b, idx = 0; p <= last; ++idx) {
        const size_t sz = (idx == 0 || nb <= 2 || p == last) ? 1 : std::min<size_t>(g, last - p);
        double rows = 0.0, rdy = 0.0;
        for (size_t q = p; q < p + sz; ++q) {
          rows += bands[q].rows;
          rdy = std::max(rdy, tile_done[(size_t)(t_first[bands[q].expert] + bands[q].rel / kTileRows)]);
        }
        tc = std::max(tc, rdy) + 2.0 * rows * (double)s->H / bw;
        p += sz;
      }
      b = last + 1;
    }
    const double total = std::max(t_prod, tc + (n_remote > 0 ? k.seg_latency_s : 0.0));
    if (total < best_t) { best_t = total; best_c = c; }
  }
  *n_consumer_cu = best_c;
  if (mgb) *mgb = g;
  if (predicted_s) *predicted_s = best_t;
  return MOE_OK;
}
