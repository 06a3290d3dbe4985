// Per-layer producer/consumer CU split (pure host function).
//
// The Weave abstract (arXiv 2609.21483) decides the split per layer from the
// routing result so that the communication and computation worker groups
// match the layer's communication/computation throughput ratio; the
// tile-signalling paper (sec. 4.3.4, Fig. 9) shows that too few consumer SMs
// leave a long transfer tail and too many slow the GEMM. The model is stated
// in partition_model.hpp; the plan kernel evaluates the same model on the
// device (MOE_CONSUMER_AUTO).
//
// Here the row tiles and segments are derived from the counts alone: row
// tiles in the GEMM's schedule order (those reaching into the remote groups
// first, experts in the band schedule's order, then the rest by expert id)
// and segments of 1, g, ..., g, 1 bands per (expert, owner) group in the band
// schedule's order, with g = the mgb returned: 2 when one band moves less
// than half a MiB (transfer bandwidth saturates only at MiB-scale transfers,
// tile-signalling paper Fig. 3(a)), else 1. The candidates are c_min,
// c_min + c_step, ... <= c_max; the step defaults to the XCD count, so a
// consumer of c = 8j CUs and a producer of n_cu - c CUs fill every XCD evenly.
#include <algorithm>
#include <vector>

#include "partition_model.hpp"

using namespace moe;

extern "C" int moe_plan_partition(const moe_shape_t* s, const int32_t* counts, const moe_calib_t* calib,
                                  int32_t* n_consumer_cu, int32_t* mgb, double* predicted_s) {
  if (s == nullptr || counts == nullptr || n_consumer_cu == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->R < 1 || s->R > MOE_MAX_RANKS || s->E < 1 || s->E % s->R != 0 || s->r_self < 0 ||
      s->r_self >= s->R || s->H < 1 || s->F < 1 || s->tb_m < 1)
    return MOE_ERR_INVALID_ARG;
  const moe_calib_t k = calib ? *calib : default_calib(256);
  if (!calib_ok(k)) return MOE_ERR_INVALID_ARG;

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
  // row tiles in schedule order: their instance time; trpos[e] = position of
  // expert e's first remote tile
  std::vector<double> tt;
  std::vector<long> trpos(El, 0);
  auto alg = [&](int e) { return (m_e[e] + tb - 1) / tb * tb; };
  auto push_tile = [&](int e, long j) {
    const long rows = std::min<long>(kModelTileRows, alg(e) - j * kModelTileRows);
    tt.push_back(model_tile_time(rows, s->F, model_rate(k, m_e[e])));
  };
  for (int e : order) {
    trpos[e] = (long)tt.size();
    for (long j = 0; j < (rb[e] * tb + kModelTileRows - 1) / kModelTileRows; ++j) push_tile(e, j);
  }
  for (int e = 0; e < El; ++e) {
    const long n = (alg(e) + kModelTileRows - 1) / kModelTileRows;
    for (long j = (rb[e] * tb + kModelTileRows - 1) / kModelTileRows; j < n; ++j) push_tile(e, j);
  }
  const long n_pos = (long)tt.size();
  // segments in schedule order: valid rows and the position of their last row tile
  const double band_bytes = 2.0 * tb * (double)s->H;
  const int g = band_bytes < 0.5 * 1048576.0 ? 2 : 1;
  std::vector<long> seg_rows, seg_pos;
  for (int e : order) {
    long rel = 0;   // first row of the group relative to the expert's base
    for (int q = 0; q < R; ++q) {
      if (q == self) continue;
      const long c = counts[e * R + q];
      const long nb = (c + tb - 1) / tb;
      const long ns = nb <= 2 ? nb : 2 + (nb - 2 + g - 1) / g;
      long j = 0;
      for (long i = 0; i < ns; ++i) {
        const long sz = (i == 0 || i == ns - 1) ? 1 : std::min<long>(g, nb - 1 - j);
        seg_rows.push_back(std::min<long>(c - j * tb, sz * tb));
        seg_pos.push_back(trpos[e] + (rel + (j + sz) * tb - 1) / kModelTileRows);
        j += sz;
      }
      rel += nb * tb;
    }
  }
  const long n_seg = (long)seg_rows.size();
  std::vector<long> rows_from(n_seg + 1, 0);   // S_i
  for (long i = n_seg - 1; i >= 0; --i) rows_from[i] = rows_from[i + 1] + seg_rows[i];

  const int tiles2 = (s->H + kModelTileCols - 1) / kModelTileCols;
  double best_t = 0.0;
  int best_c = -1;
  std::vector<double> wend;
  for (int c = k.c_min; c <= k.c_max; c += k.c_step) {
    const long P = k.n_cu - c;
    const long n_inst = n_pos * tiles2;
    const long n_waves = (n_inst + P - 1) / P;
    wend.assign((size_t)n_waves, 0.0);
    double t = 0.0;
    for (long w = 0; w < n_waves; ++w) {
      long p0, p1;
      model_wave_span(w, P, tiles2, n_pos, &p0, &p1);
      double len = 0.0;
      for (long q = p0; q <= p1; ++q) len = std::max(len, tt[(size_t)q]);
      t = model_wave_end(t, len, std::min(P, n_inst - w * P), P);
      wend[(size_t)w] = t;
    }
    const double bw = model_copy_bw(k, c);
    double tc = 0.0;
    for (long i = 0; i < n_seg; ++i)
      tc = std::max(tc, model_copy_end(wend[(size_t)((seg_pos[i] * tiles2 + tiles2 - 1) / P)], rows_from[i],
                                       s->H, bw));
    const double total = model_total(t, tc, n_seg > 0, k.seg_latency_s);
    if (best_c < 0 || total < best_t) { best_t = total; best_c = c; }
  }
  *n_consumer_cu = best_c;
  if (mgb) *mgb = g;
  if (predicted_s) *predicted_s = best_t;
  return MOE_OK;
}
