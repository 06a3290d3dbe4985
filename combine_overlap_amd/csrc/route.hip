// Step 1 of the MoE forward ("Routing", sec. 2.1 of the tile-signalling
// overlap paper): per token, the top-k experts by logit and their gates,
// plus the per-(local expert, source rank) row counts that the dispatch
// delivers to this rank.
//
// k_route: one routing group of G lanes (the fewest with at most 32 logits
// each: G = 8 for 256 experts, 1 up to 32) owns a token; lane i of the group
// holds the logits of experts i NQ ... i NQ + NQ - 1 as order-preserving
// integer keys (loaded 16 bytes at a time when E is a multiple of 4). Each of the k rounds takes the lane's best key by a tournament, then
// the group's best by a butterfly (higher logit wins, equal logits go to the
// lower expert id), and the winner's key drops to 0 (below every logit).
// The width balances the per-token instruction count (vector-ALU issue
// bound) against enough waves per SIMD to hide each wave's dependency chain.
// The grid covers the tokens (a workgroup holds 256 / G of them), so every
// CU has many tokens' loads in flight.
//
// k_chunk_hist: per routing chunk (kChunk tokens of one source rank), how
// many of its (token, slot) pairs chose each local expert; its last block
// turns the chunk histograms into counts[e][s] and each chunk's first row
// inside its (e, s) group (the index ranks rows by token inside a group).
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 256;

// order-preserving unsigned key of a float (larger key = larger value; -0 is
// taken as +0); 0 is below every key and marks "not a candidate"
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // negative: all bits flipped
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int G, int NQ>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ logits,
                                                          int32_t* __restrict__ ids_out,
                                                          float* __restrict__ gates_out,
                                                          int32_t* __restrict__ hist_arrivals,
                                                          int n_tok, int E, int k, int gate_kind) {
  // the next launch's arrival counter (k_chunk_hist) starts from zero
  if (blockIdx.x == 0 && threadIdx.x == 0) *hist_arrivals = 0;
  const int lane = threadIdx.x & 63;
  const int gi = lane & (G - 1);                         // lane inside the routing group
  constexpr int per_block = kRouteThreads / G;
  const int g_tok = blockIdx.x * per_block + (int)threadIdx.x / G;
  const bool active = g_tok < n_tok;
  const size_t g = active ? (size_t)g_tok : 0;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(logits) + g * E;
  // keys of experts gi NQ + q: unconditional loads with clamped indices
  // (predicated ones would each wait for the previous), then the selection
  const int e0 = gi * NQ;
  uint32_t key[NQ];
  if ((E & 3) == 0) {
    // rows are 16-byte aligned; a 4-expert chunk is wholly inside or past E
    const u32x4* row4 = reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int c = 0; c < NQ / 4; ++c) {
      const int i4 = (e0 >> 2) + c;
      const u32x4 v = row4[i4 < (E >> 2) ? i4 : 0];
#pragma unroll
      for (int j = 0; j < 4; ++j) key[4 * c + j] = v[j];
    }
  } else {
#pragma unroll
    for (int q = 0; q < NQ; ++q) key[q] = row[min(e0 + q, E - 1)];
  }
  // (an inactive token's group reads row 0 and writes nothing; experts past E get key 0)
#pragma unroll
  for (int q = 0; q < NQ; ++q) key[q] = order_key(key[q]) & (0u - (uint32_t)(e0 + q < E));
  uint32_t sel_k[16];
  int sel_id[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    // best of this lane: a tournament over q in which the right entry replaces
    // the left only if strictly larger, so the lower q (lower id) wins ties
    uint32_t tk[NQ];
    int tq[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) { tk[q] = key[q]; tq[q] = q; }
#pragma unroll
    for (int st = 1; st < NQ; st <<= 1)
#pragma unroll
      for (int q = 0; q + st < NQ; q += 2 * st)
        if (tk[q + st] > tk[q]) { tk[q] = tk[q + st]; tq[q] = tq[q + st]; }
    uint32_t bk = tk[0];
    int bid = e0 + tq[0];
#pragma unroll
    for (int off = G >> 1; off > 0; off >>= 1) {   // across the group: larger key, then lower id
      const uint32_t ok = __shfl_xor(bk, off, G);
      const int oid = __shfl_xor(bid, off, G);
      if (ok > bk || (ok == bk && oid < bid)) { bk = ok; bid = oid; }
    }
    const int wq = (bid / NQ == gi) ? bid - e0 : -1;   // the winner leaves the candidates
#pragma unroll
    for (int q = 0; q < NQ; ++q) key[q] = (q == wq) ? 0u : key[q];
    sel_k[r] = bk;
    sel_id[r] = bid;
  }
  if (!active) return;
  // gates over the k selected logits (fp32)
  float w[16];
  float sum = 0.f;
  const float v0 = key_value(sel_k[0]);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    const float v = key_value(sel_k[r]);
    float x;
    if (gate_kind == MOE_GATE_SOFTMAX) x = expf(v - v0);
    else x = 1.0f / (1.0f + expf(-v));
    w[r] = x;
    sum += x;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r >= k) break;
    if ((r & (G - 1)) == gi) {   // G may be smaller than k: lane gi writes selections gi, gi + G, ...
      ids_out[g * k + r] = sel_id[r];
      gates_out[g * k + r] = w[r] / sum;
    }
  }
}

// Per chunk: the local-expert histogram of its tokens' selected ids. The
// last block to finish (an arrival counter that k_route zeroed) then turns
// the chunk histograms into counts[e][s] and each chunk's first row inside
// its (e, s) group (the index ranks rows by token inside a group): one
// launch instead of a histogram launch and a one-workgroup count launch.
__global__ __launch_bounds__(256) void k_chunk_hist(const int32_t* __restrict__ ids, int32_t* __restrict__ chunk_counts,
                                                     int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ arrivals, int T, int k, int R, int El,
                                                     int first_local, int chunks_per_rank) {
  __shared__ int cnt[kPlanMaxElRoute];
  __shared__ int s_last;
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
  // device-scope stores: they write through this XCD's L2, so the last block
  // (on any XCD) reads them with device-scope loads once it has seen every
  // arrival, which each block counts after its stores have completed
  for (int i = threadIdx.x; i < El; i += blockDim.x)
    __hip_atomic_store(chunk_counts + chunk * El + i, cnt[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(arrivals, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  // counts[e][s] and the exclusive per-chunk row offsets inside each (e, s) group
  for (int pp = threadIdx.x; pp < El * R; pp += blockDim.x) {
    const int e = pp / R, q = pp % R;
    int acc = 0;
    for (int c0 = 0; c0 < chunks_per_rank; c0 += 8) {   // 8 loads in flight, then the 8 stores
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = c0 + u < chunks_per_rank
                   ? __hip_atomic_load(chunk_counts + (q * chunks_per_rank + c0 + u) * El + e, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < chunks_per_rank) chunk_base[(q * chunks_per_rank + c0 + u) * El + e] = acc;
        acc += v[u];
      }
    }
    counts[e * R + q] = acc;
  }
}

hipError_t launch_route(const Geometry& g, const float* logits, int32_t* ids, float* gates,
                        const moe_plan_t& p, hipStream_t st) {
  // group width: the fewest lanes with at most 32 logits each (E <= 512: G <= 16)
  int G = 1;
  while (G * 32 < g.E) G <<= 1;
  int NQ = 8;
  while (NQ * G < g.E) NQ <<= 1;
  const int n_tok = g.R * g.T;
  const int per_block = kRouteThreads / G;
  dim3 grid((n_tok + per_block - 1) / per_block), block(kRouteThreads);
#define MOE_ROUTE_CASE(GG, QQ)                                                                 \
  if (G == GG && NQ == QQ) {                                                                   \
    hipLaunchKernelGGL((k_route<GG, QQ>), grid, block, 0, st, logits, ids, gates, p.meta + META_HISTCTR, \
                       n_tok, g.E, g.k, g.gate_kind);                                          \
    return hipGetLastError();                                                                  \
  }
  MOE_ROUTE_CASE(1, 8)
  MOE_ROUTE_CASE(1, 16)
  MOE_ROUTE_CASE(1, 32)
  MOE_ROUTE_CASE(2, 32)
  MOE_ROUTE_CASE(4, 32)
  MOE_ROUTE_CASE(8, 32)
  MOE_ROUTE_CASE(16, 32)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_count(const Geometry& g, const int32_t* ids, int32_t* counts, const moe_plan_t& p,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_hist, dim3(g.n_chunks), dim3(256), 0, st, ids, p.chunk_counts, p.chunk_base, counts,
                     p.meta + META_HISTCTR, g.T, g.k, g.R, g.El, g.r_self * g.El, g.chunks_per_rank);
  return hipGetLastError();
}

}  // namespace moe
