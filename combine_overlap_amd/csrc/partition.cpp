// Per-layer producer/consumer CU split (pure host function).
//
// The Weave abstract (arXiv 2609.21483) decides the split per layer from the
// routing result so that the communication and computation worker groups
// match the layer's communication/computation throughput ratio; the
// tile-signalling paper (sec. 4.3.4, Fig. 9) shows that too few consumer SMs
// leave a long transfer tail and too many slow the GEMM.
//
// Model (the form is not given on the pages; this is the plainest one that
// uses only the routing counts and two measured rates):
//   P(c)  = n_cu - c producer CUs
//   T_g   = sum_e flops2_e / (rate(M_e) * P(c))      overlapped output projection
//           flops2_e = 2 * H * F * padded rows of expert e,
//           rate(M) = gemm_flops_per_cu * M / (M + gemm_m_half)
//   BW(c) = min(c * copy_bw_per_cu, copy_bw_max)       bytes moved per second
//   T_c   = remote_bytes / BW(c) + n_seg * seg_latency
//   t_1   = first band ready: one tile of the output projection on one CU
//   t_end = last segment (one band) after the producer finishes
//   T(c)  = max(T_g, t_1 + T_c) + band_bytes / BW(c)
// c = argmin T(c) over [c_min, c_max] (smallest c on ties). mgb = 2 when a
// single band moves less than half a MiB (the bandwidth curve of the
// tile-signalling paper, Fig. 3(a), saturates only at MiB-scale transfers),
// else 1.
#include <math.h>
#include <stdint.h>

#include "moe_overlap.h"

extern "C" int moe_plan_partition(const moe_shape_t* s, const int32_t* counts, const moe_calib_t* calib,
                                  int32_t* n_consumer_cu, int32_t* mgb, double* predicted_s) {
  if (s == nullptr || counts == nullptr || n_consumer_cu == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->R < 1 || s->R > MOE_MAX_RANKS || s->E < 1 || s->E % s->R != 0 || s->r_self < 0 ||
      s->r_self >= s->R || s->H < 1 || s->F < 1 || s->tb_m < 1)
    return MOE_ERR_INVALID_ARG;
  moe_calib_t c0;
  c0.gemm_flops_per_cu = 2.5e15 / 256.0 * 0.6;
  c0.gemm_m_half = 64.0;
  c0.copy_bw_per_cu = 60e9;
  c0.copy_bw_max = 2.5e12;
  c0.seg_latency_s = 2e-6;
  c0.n_cu = 256;
  c0.c_min = 2;
  c0.c_max = 16;
  const moe_calib_t& k = calib ? *calib : c0;
  if (k.n_cu < 2 || k.c_min < 1 || k.c_max < k.c_min || k.c_max >= k.n_cu || k.gemm_flops_per_cu <= 0 ||
      k.copy_bw_per_cu <= 0 || k.copy_bw_max <= 0 || k.gemm_m_half < 0 || k.seg_latency_s < 0)
    return MOE_ERR_INVALID_ARG;

  const int El = s->E / s->R, R = s->R, tb = s->tb_m;
  double flops_work = 0.0;   // sum_e flops2_e / rate(M_e)   (CU-seconds)
  double remote_rows = 0.0;
  long n_seg_bands = 0;
  for (int e = 0; e < El; ++e) {
    long m = 0;
    for (int q = 0; q < R; ++q) {
      const long c = counts[e * R + q];
      if (c < 0) return MOE_ERR_INVALID_ARG;
      if (q != s->r_self) {
        m += (c + tb - 1) / tb * tb;
        remote_rows += (double)c;
        n_seg_bands += (c + tb - 1) / tb;
      } else {
        m += c;
      }
    }
    const long mp = (m + tb - 1) / tb * tb;
    if (mp == 0) continue;
    const double fl = 2.0 * s->H * (double)s->F * (double)mp;
    const double rate = k.gemm_flops_per_cu * (double)m / ((double)m + k.gemm_m_half);
    flops_work += fl / rate;
  }
  const double band_bytes = 2.0 * tb * (double)s->H;
  const int g = band_bytes < 0.5 * 1048576.0 ? 2 : 1;
  const double remote_bytes = 2.0 * (double)s->H * remote_rows;
  // segments: 1 + ceil((nb-2)/g) + 1 per group, approximated from the band total
  const double n_seg = g == 1 ? (double)n_seg_bands : 0.5 * (double)n_seg_bands + 1.0;
  const double t_tile = 2.0 * tb * 256.0 * (double)s->F / k.gemm_flops_per_cu;
  double best_t = INFINITY;
  int best_c = k.c_min;
  for (int c = k.c_min; c <= k.c_max; ++c) {
    const double bw = fmin(c * k.copy_bw_per_cu, k.copy_bw_max);
    const double tg = flops_work / (double)(k.n_cu - c);
    const double tc = remote_bytes / bw + n_seg * k.seg_latency_s;
    const double tail = remote_rows > 0 ? band_bytes / bw : 0.0;
    const double t = fmax(tg, (remote_rows > 0 ? t_tile : 0.0) + tc) + tail;
    if (t < best_t) { best_t = t; best_c = c; }
  }
  *n_consumer_cu = best_c;
  if (mgb) *mgb = g;
  if (predicted_s) *predicted_s = best_t;
  return MOE_OK;
}
