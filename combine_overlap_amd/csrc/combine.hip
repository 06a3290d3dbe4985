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

// Sum of one 16-byte column step of N rows, rounded once to bf16.
template <int N>
__device__ __forceinline__ u32x4 weigh(const u32x4* d, const float* w) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] += w[i] * __uint_as_float(d[i][c] << 16);
      acc[2 * c + 1] += w[i] * __uint_as_float(d[i][c] & 0xffff0000u);
    }
  u32x4 o;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    o[c] = (uint32_t)f32_to_bf16_rne(acc[2 * c]) | ((uint32_t)f32_to_bf16_rne(acc[2 * c + 1]) << 16);
  return o;
}

// One token's row: the N slots in `mask` (ascending j) are summed with their
// gates. N is a compile-time constant, so the row pointers and gates stay in
// registers. U column steps are loaded before any is reduced, so about eight
// 16-byte loads per lane are in flight whatever N is (one wave per token
// would otherwise wait out a full memory latency per step when N is 1).
template <int N>
__device__ __forceinline__ void combine_token(const uint16_t* base, const float* __restrict__ gates,
                                              const int32_t* __restrict__ recv_row, size_t g, int k,
                                              uint32_t mask, u32x4* dst, int H, int lane) {
  constexpr int NN = N > 0 ? N : 1;
  constexpr int U = N >= 8 ? 1 : (N == 0 ? 1 : 8 / N);
  const u32x4* rows[NN];
  float w[NN];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = __builtin_ctz(mask);   // i-th local slot
    mask &= mask - 1;
    rows[i] = reinterpret_cast<const u32x4*>(base + (size_t)recv_row[g * k + j] * H);
    w[i] = gates[g * k + j];
  }
  const int nv = H / 8;
  int v = lane;
  for (; v + (U - 1) * 64 < nv; v += U * 64) {
    u32x4 d[U][NN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < N; ++i) d[u][i] = rows[i][v + u * 64];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[v + u * 64] = weigh<N>(d[u], w);
  }
  for (; v < nv; v += 64) {
    u32x4 d[NN];
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = rows[i][v];
    dst[v] = weigh<N>(d, w);
  }
}

template <int N, int KMAX>
__device__ __forceinline__ void combine_dispatch(int n, const uint16_t* base, const float* gates,
                                                 const int32_t* recv_row, size_t g, int k, uint32_t mask,
                                                 u32x4* dst, int H, int lane) {
  if constexpr (N <= KMAX) {
    if (n == N) {
      combine_token<N>(base, gates, recv_row, g, k, mask, dst, H, lane);
      return;
    }
    combine_dispatch<N + 1, KMAX>(n, base, gates, recv_row, g, k, mask, dst, H, lane);
  }
}

// KMAX >= k. A token's local slots are found first (recv_row >= 0; the same
// for the whole wave), and the row loop is specialised on their count, so a
// token reads only its local rows: with k = 8 of 256 experts and 32 local,
// most tokens have one local slot of eight.
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(BufPtrs bufs, const uint16_t* __restrict__ y,
                                                  const float* __restrict__ gates,
                                                  const int32_t* __restrict__ recv_row,
                                                  uint16_t* __restrict__ out, int n_tok, int T,
                                                  int H, int k, int r_self) {
  // the token index is the same across the wave: held in a scalar register,
  // so the slot scan below uses scalar loads and the dispatch scalar branches
  const int g = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (g >= n_tok) return;
  const int s = g / T;
  const uint16_t* base = (s == r_self) ? y : bufs.p[s];
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k && recv_row[(size_t)g * k + j] >= 0) mask |= 1u << j;
  const int n = __builtin_popcount(mask);
  combine_dispatch<0, KMAX>(n, base, gates, recv_row, (size_t)g, k, mask,
                            reinterpret_cast<u32x4*>(out + (size_t)g * H), H, lane);
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
