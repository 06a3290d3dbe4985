// The transfer's host-side setup and the baseline's bulk copy.
//
// The consumer of the tile-signalling overlap paper (sec. 3.3.2-3.3.3) is the
// device function consume() (consumer.hpp), run by the first c workgroups of
// the overlapped output projection; consumer_args() packs its arguments.
//
// The bulk copy (the non-overlapped baseline's second all-to-all, sec. 4.1.3)
// copies all segments after the producer has finished, using every CU.
#include "consumer.hpp"

namespace moe {

#ifndef MOE_COPY_UNROLL
#define MOE_COPY_UNROLL 8
#endif

// plain 16-byte loads and stores, MOE_COPY_UNROLL loads in flight per thread.
// Streaming (non-temporal) stores cost 15-20% here: 87 against 72 us for
// the 209 MB of remote rows at H = 7168 (MI355X, same box).
__device__ __forceinline__ void copy_units(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                           size_t lo, size_t hi, int tid, int nthr) {
  constexpr int U = MOE_COPY_UNROLL;
  size_t i = lo + tid;
  for (; i + (U - 1) * (size_t)nthr < hi; i += U * (size_t)nthr) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * (size_t)nthr];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * (size_t)nthr] = v[u];
  }
  for (; i < hi; i += nthr) dst[i] = src[i];
}

// baseline: all remote segments after the producer, on all CUs. The segments
// are cut into 64 KiB copy units (prefix in seg_unit0); workgroups take units
// grid-stride and find their segment by binary search.
__global__ __launch_bounds__(256) void k_bulk_copy(const uint16_t* __restrict__ y, BufPtrs bufs,
                                                    moe_plan_t p, int H) {
  const int n_seg = p.meta[META_NSEG];
  const int n_units = p.meta[META_NUNITS];
  constexpr size_t kUnit16 = kCopyUnitBytes / 16;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    int lo = 0, hi = n_seg - 1;
    while (lo < hi) {   // last segment whose first unit is <= u
      const int mid = (lo + hi + 1) >> 1;
      if (p.seg_unit0[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int sgi = lo;
    const size_t units16 = (size_t)p.seg_rows[sgi] * H / 8;
    const size_t a = (size_t)(u - p.seg_unit0[sgi]) * kUnit16;
    const size_t b = a + kUnit16 < units16 ? a + kUnit16 : units16;
    const u32x4* src = reinterpret_cast<const u32x4*>(y + (size_t)p.seg_src_row[sgi] * H);
    u32x4* dst = reinterpret_cast<u32x4*>(bufs.p[p.seg_dest[sgi]] + (size_t)p.seg_dst_row[sgi] * H);
    copy_units(src, dst, a, b, threadIdx.x, 256);
  }
}

ConsumerArgs consumer_args(const Geometry& g, const uint16_t* y, BufPtrs bufs, const moe_plan_t& p,
                           const uint32_t* flags, uint32_t epoch, uint64_t* trace, uint64_t wait_ticks) {
  ConsumerArgs c{};
  c.y = y;
  c.bufs = bufs;
  c.meta = p.meta;
  c.seg_unit0 = p.seg_unit0;
  c.seg_rows = p.seg_rows;
  c.seg_src_row = p.seg_src_row;
  c.seg_dst_row = p.seg_dst_row;
  c.seg_dest = p.seg_dest;
  c.seg_tile0 = p.seg_tile0;
  c.seg_tile1 = p.seg_tile1;
  c.flags = flags;
  c.epoch = epoch;
  c.trace = trace;
  c.trace_seg = 8 + g.max_flags;
  c.tiles2 = g.tiles2;
  c.H = g.H;
  c.wait_ticks = wait_ticks;
  return c;
}

hipError_t launch_bulk_copy(const Geometry& g, const uint16_t* y, BufPtrs bufs,
                            const moe_plan_t& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_bulk_copy, dim3(grid), dim3(256), 0, st, y, bufs, p, g.H);
  return hipGetLastError();
}

}  // namespace moe
