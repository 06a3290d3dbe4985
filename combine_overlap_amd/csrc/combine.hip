// Weighted reduction ("scale", sec. 2.1 step 5 of the tile-signalling
// overlap paper): for every token (s, t) the owner sums gate * returned
// expert row over the token's slots (ascending j) whose expert is local to
// this rank. Rows come from combine_buf[s] for remote owners and straight
// from y_perm for the local owner. fp32 accumulation, one bf16 rounding.
//
// One wave per token; each lane handles 8 consecutive bf16 (16 bytes) per
// step, so every row is read with fully coalesced 16-byte loads.
#include "common.hpp"

namespace moe {

// KMAX >= k: the slot loop is unrolled (row pointers and gates stay in
// registers, every slot's load of a step is in flight at once); slots whose
// expert is not local carry a zero gate and read row 0 of y, so the
// accumulation order is still ascending j.
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(BufPtrs bufs, const uint16_t* __restrict__ y,
                                                  const float* __restrict__ gates,
                                                  const int32_t* __restrict__ recv_row,
                                                  uint16_t* __restrict__ out, int n_tok, int T,
                                                  int H, int k, int r_self) {
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= n_tok) return;
  const int s = g / T;
  const uint16_t* base = (s == r_self) ? y : bufs.p[s];
  const u32x4* rows[KMAX];
  float w[KMAX];
  bool on[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int r = j < k ? recv_row[(size_t)g * k + j] : -1;
    on[j] = r >= 0;
    rows[j] = reinterpret_cast<const u32x4*>(on[j] ? base + (size_t)r * H : y);
    w[j] = on[j] ? gates[(size_t)g * k + j] : 0.f;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)g * H);
  const int nv = H / 8;
  for (int v = lane; v < nv; v += 64) {
    u32x4 d[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) d[j] = rows[j][v];   // unconditional: keeps the loads in flight together
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (!on[j]) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] += w[j] * __uint_as_float(d[j][c] << 16);
        acc[2 * c + 1] += w[j] * __uint_as_float(d[j][c] & 0xffff0000u);
      }
    }
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = (uint32_t)f32_to_bf16_rne(acc[2 * c]) | ((uint32_t)f32_to_bf16_rne(acc[2 * c + 1]) << 16);
    dst[v] = o;
  }
}

hipError_t launch_combine(const Geometry& g, BufPtrs bufs, const uint16_t* y, const float* gates,
                          const moe_plan_t& p, uint16_t* out, hipStream_t st) {
  const int n_tok = g.R * g.T;
  const dim3 grid((n_tok + 3) / 4), block(256);
#define MOE_COMBINE_CASE(N)                                                                       \
  if (g.k <= N) {                                                                                 \
    hipLaunchKernelGGL(k_combine<N>, grid, block, 0, st, bufs, y, gates, p.recv_row, out, n_tok, g.T, \
                       g.H, g.k, g.r_self);                                                       \
    return hipGetLastError();                                                                     \
  }
  MOE_COMBINE_CASE(2)
  MOE_COMBINE_CASE(4)
  MOE_COMBINE_CASE(8)
  MOE_COMBINE_CASE(16)
#undef MOE_COMBINE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
