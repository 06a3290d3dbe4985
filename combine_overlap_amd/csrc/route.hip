// Step 1 of the MoE forward ("Routing", sec. 2.1 of the tile-signalling
// overlap paper): per token, the top-k experts by logit and their gates,
// plus the per-(local expert, source rank) row counts that the dispatch
// delivers to this rank.
//
// k_route: one routing group of G lanes (G = the smallest power of two with
// 8 G >= E) owns a token; lane i of the group holds logits i, i+G, i+2G, ...
// (at most 8). Each of the k rounds is a butterfly arg-max inside the group
// (higher logit wins, equal logits go to the lower expert id) followed by
// masking the winner. Small groups keep the butterfly short and put many
// tokens in each wave.
// The grid covers the tokens (a workgroup holds 256 / G of them), so every
// CU has many tokens' loads in flight.
//
// k_chunk_hist: per routing chunk (kChunk tokens of one source rank), how
// many of its (token, slot) pairs chose each local expert; k_count turns the
// chunk histograms into counts[e][s] and each chunk's first row inside its
// (e, s) group (the gather ranks rows by token inside a group).
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 256;

template <int NQ>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ logits,
                                                          int32_t* __restrict__ ids_out,
                                                          float* __restrict__ gates_out,
                                                          int n_tok, int E, int k, int G,
                                                          int gate_kind) {
  const int lane = threadIdx.x & 63;
  const int gi = lane % G;                               // lane inside the routing group
  const int per_block = kRouteThreads / G;
  const int g_tok = blockIdx.x * per_block + (int)threadIdx.x / G;
  const bool active = g_tok < n_tok;
  const size_t g = active ? (size_t)g_tok : 0;
  float v[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = gi + q * G;
    v[q] = (active && e < E) ? logits[g * E + e] : -INFINITY;
  }
  uint32_t taken = 0;
  float sel_v[16];
  int sel_id[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    // best of this lane: ids rise with q, so a strict '>' keeps the lowest id among equals
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = gi + q * G;
      if (e < E && !(taken >> q & 1u) && (bid == 0x7fffffff || v[q] > bv)) { bv = v[q]; bid = e; }
    }
    for (int off = G >> 1; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, G);
      const int oid = __shfl_xor(bid, off, G);
      if (ov > bv || (ov == bv && oid < bid)) { bv = ov; bid = oid; }
    }
    if (bid % G == gi) taken |= 1u << (bid / G);
    sel_v[r] = bv;
    sel_id[r] = bid;
  }
  if (!active) return;
  // gates over the k selected logits (fp32)
  float w[16];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    float x;
    if (gate_kind == MOE_GATE_SOFTMAX) x = expf(sel_v[r] - sel_v[0]);
    else x = 1.0f / (1.0f + expf(-sel_v[r]));
    w[r] = x;
    sum += x;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    if (r % G == gi) {   // G may be smaller than k: lane gi writes selections gi, gi + G, ...
      ids_out[g * k + r] = sel_id[r];
      gates_out[g * k + r] = w[r] / sum;
    }
  }
}

// per chunk: local-expert histogram of its tokens' selected ids
__global__ __launch_bounds__(256) void k_chunk_hist(const int32_t* __restrict__ ids,
                                                     int32_t* __restrict__ chunk_counts, int T, int k,
                                                     int El, int first_local, int chunks_per_rank) {
  __shared__ int cnt[kPlanMaxElRoute];
  const int chunk = blockIdx.x;
  const int s = chunk / chunks_per_rank;
  const int t0 = (chunk % chunks_per_rank) * kChunk;
  const int t1 = min(T, t0 + kChunk);
  for (int i = threadIdx.x; i < El; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const size_t base = ((size_t)s * T + t0) * k;
  const int n = (t1 - t0) * k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int el = ids[base + i] - first_local;
    if (el >= 0 && el < El) atomicAdd(&cnt[el], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < El; i += blockDim.x) chunk_counts[chunk * El + i] = cnt[i];
}

// counts[e][s] and the exclusive per-chunk row offsets inside each (e, s) group
__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ chunk_counts,
                                                int32_t* __restrict__ chunk_base,
                                                int32_t* __restrict__ counts, int R, int El,
                                                int chunks_per_rank) {
  for (int p = threadIdx.x; p < El * R; p += blockDim.x) {
    const int e = p / R, s = p % R;
    int acc = 0;
    for (int c = 0; c < chunks_per_rank; ++c) {
      const int ch = s * chunks_per_rank + c;
      chunk_base[ch * El + e] = acc;
      acc += chunk_counts[ch * El + e];
    }
    counts[e * R + s] = acc;
  }
}

hipError_t launch_route(const Geometry& g, const float* logits, int32_t* ids, float* gates,
                        const moe_plan_t& p, hipStream_t st) {
  (void)p;
  int G = 1;
  while (G * 8 < g.E) G <<= 1;   // E <= 512: G <= 64
  const int nq = (g.E + G - 1) / G;
  const int n_tok = g.R * g.T;
  const int per_block = kRouteThreads / G;
  dim3 grid((n_tok + per_block - 1) / per_block), block(kRouteThreads);
#define MOE_ROUTE_CASE(N)                                                                     \
  if (nq <= N) {                                                                              \
    hipLaunchKernelGGL(k_route<N>, grid, block, 0, st, logits, ids, gates, n_tok, g.E, g.k, G, \
                       g.gate_kind);                                                          \
    return hipGetLastError();                                                                 \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_count(const Geometry& g, const int32_t* ids, int32_t* counts, const moe_plan_t& p,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_hist, dim3(g.n_chunks), dim3(256), 0, st, ids, p.chunk_counts, g.T, g.k,
                     g.El, g.r_self * g.El, g.chunks_per_rank);
  hipLaunchKernelGGL(k_count, dim3(1), dim3(256), 0, st, p.chunk_counts, p.chunk_base, counts,
                     g.R, g.El, g.chunks_per_rank);
  return hipGetLastError();
}

}  // namespace moe
