// Arithmetic of the per-layer producer/consumer CU-split model, shared by the
// host function moe_plan_partition and its evaluation on the device inside
// the plan kernel. Both sides evaluate the same closed form with the same
// operations in the same order (no contraction into fused multiply-adds),
// so they predict bit-identical times and pick the same c.
//
// The model (its form is not given on the pages; this is the plainest one
// that uses only the routing counts and measured rates), for c consumer CUs:
//  * the output projection runs on P = n_cu - c CUs. Its row tiles (up to 256
//    rows of one expert's tb_m-aligned rows, K = F) are taken in schedule
//    order, each with tiles2 column tiles of 256; a tile instance takes
//    t_tile = 2 rows32 256 F / rate(M_e) on one CU (rows32 = its rows rounded
//    up to 32, rate(M) = gemm_flops_per_cu M / (M + gemm_m_half));
//  * the instances run in waves of P: a wave lasts as long as its slowest
//    instance, a partial last wave of n instances max(n / P, 1/3) of that
//    (fewer tiles share the memory bandwidth), and a row tile is ready when
//    the wave holding its last column tile ends;
//  * the consumer copies the segments in schedule order, each once its row
//    tiles are ready and the previous copy is done, at
//    BW(c) = c b / (1 + c b / B) (b = copy_bw_per_cu, B = copy_bw_max: linear
//    in c for few CUs, saturating at what the copy reaches beside the GEMM),
//    plus seg_latency_s once. With ready_i and the valid rows S_i of segments
//    i, i+1, ..., the copy ends at max_i (ready_i + 2 H S_i / BW(c));
//  * T(c) = max(producer end, copy end); c = argmin over the candidates,
//    the smallest c on ties.
#pragma once

#include <stdint.h>

#include "moe_overlap.h"

namespace moe {

constexpr int kModelTileRows = 256;   // GEMM row-tile height
constexpr int kModelTileCols = 256;   // output-projection column tile

// calibration measured on MI355X: 3.6-4.4 TFLOP/s per producer CU on the
// output projection; b, B and the copy's tail fitted to the measured best c
// of 76 shapes (the Table-2 grid of the tile-signalling paper at N = 4096 and
// 8192, and the 16 layers of the dynamic-split workload): BW(c) = 133, 229,
// 356, 436 GB/s at c = 8, 16, 32, 48, plus 30 us for the last batch
inline moe_calib_t default_calib(int n_cu) {
  moe_calib_t k;
  k.gemm_flops_per_cu = 3.5e12;
  k.gemm_m_half = 0.0;
  k.copy_bw_per_cu = 20e9;
  k.copy_bw_max = 800e9;
  k.seg_latency_s = 30e-6;
  k.n_cu = n_cu;
  k.c_max = n_cu - 1 < 48 ? n_cu - 1 : 48;
  k.c_min = k.c_max < 8 ? (k.c_max > 1 ? k.c_max : 1) : 8;
  k.c_step = 8;
  return k;
}

__host__ __device__ inline double model_rate(const moe_calib_t& k, long m) {
#pragma clang fp contract(off)
  const double mm = (double)(m > 1 ? m : 1);
  return k.gemm_flops_per_cu * mm / (mm + k.gemm_m_half);
}

// one instance of a row tile with `rows` rows
__host__ __device__ inline double model_tile_time(long rows, int F, double rate) {
#pragma clang fp contract(off)
  return 2.0 * (double)((rows + 31) / 32 * 32) * (double)kModelTileCols * (double)F / rate;
}

// wave end after a wave of `len` holding n of P instances (I: long on the
// host, int in the plan kernel, whose values fit; both give the same doubles)
template <typename I>
__host__ __device__ inline double model_wave_end(double t, double len, I n, I P) {
#pragma clang fp contract(off)
  if (n >= P) return t + len;
  const double f = (double)n / (double)P;
  return t + len * (f > 1.0 / 3.0 ? f : 1.0 / 3.0);
}

__host__ __device__ inline double model_copy_bw(const moe_calib_t& k, int c) {
#pragma clang fp contract(off)
  return (double)c * k.copy_bw_per_cu / (1.0 + (double)c * k.copy_bw_per_cu / k.copy_bw_max);
}

// copy end if segment i (ready at `ready`) and the S_i rows from it on are copied last
__host__ __device__ inline double model_copy_end(double ready, long rows_from_i, int H, double bw) {
#pragma clang fp contract(off)
  return ready + 2.0 * (double)rows_from_i * (double)H / bw;
}

__host__ __device__ inline double model_total(double t_prod, double t_copy, bool any_copy, double latency) {
#pragma clang fp contract(off)
  const double tc = any_copy ? t_copy + latency : 0.0;
  return t_prod > tc ? t_prod : tc;
}

// positions of row tiles covered by wave w of P instances (tiles2 per row tile)
template <typename I>
__host__ __device__ inline void model_wave_span(I w, I P, int tiles2, I n_pos, I* p0, I* p1) {
  *p0 = w * P / tiles2;
  const I last = ((w + 1) * P - 1) / tiles2;
  *p1 = last < n_pos - 1 ? last : n_pos - 1;
}

__host__ __device__ inline bool calib_ok(const moe_calib_t& k) {
  return k.n_cu >= 2 && k.c_min >= 1 && k.c_max >= k.c_min && k.c_max < k.n_cu && k.c_step >= 1 &&
         k.gemm_flops_per_cu > 0 && k.copy_bw_per_cu > 0 && k.copy_bw_max > 0 && k.gemm_m_half >= 0 &&
         k.seg_latency_s >= 0;
}

}  // namespace moe
