// Consumer of the tile-signalling overlap paper (sec. 3.3.2-3.3.3): a
// persistent kernel on a small set of CUs that walks the transfer segments
// in schedule order, waits until every tile of a segment's row bands carries
// the current epoch flag (acquire loads at agent scope), and then moves the
// segment's valid rows with one contiguous copy into the combine buffer of
// the owner rank. Flags and rows are read with device-scope loads, which
// pair with the producer's device-scope stores and completion wait (see the
// output-projection epilogue); no L2 invalidate is issued per segment. On one GPU the owner's receive buffer is a buffer in local
// HBM; the copy is split evenly across the c consumer workgroups.
//
// Each consumer workgroup (1024 threads) also reserves enough LDS that no
// producer workgroup can share its CU, which keeps the two partitions
// disjoint (sec. 2.4: persistent kernels with fixed workgroup counts).
//
// Every wait is bounded: after kWaitTicks of the 100 MHz constant clock the
// device status word becomes MOE_ERR_TIMEOUT and all consumer workgroups exit.
//
// The bulk copy (the non-overlapped baseline's second all-to-all, sec. 4.1.3)
// copies all segments after the producer has finished, using every CU.
#include "common.hpp"

namespace moe {

constexpr uint64_t kWaitTicks = 200000000ull;   // 2 s at 100 MHz
constexpr int kConsumerThreads = 1024;
constexpr int kConsumerLdsBytes = 80 * 1024;

#ifndef MOE_DEVICE_SCOPE_PUBLISH
#define MOE_DEVICE_SCOPE_PUBLISH 1
#endif

#ifndef MOE_COPY_UNROLL
#define MOE_COPY_UNROLL 8
#endif

// plain 16-byte loads (non-temporal loads halve the per-CU rate), streaming
// stores; MOE_COPY_UNROLL loads in flight per thread
template <bool DEVICE_SCOPE>
__device__ __forceinline__ void copy_units(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                           size_t lo, size_t hi, int tid, int nthr) {
  constexpr int U = MOE_COPY_UNROLL;
  auto ld = [&](size_t i) -> u32x4 {
    if constexpr (DEVICE_SCOPE) {
      // device-scope (sc1) loads miss in this XCD's L2 unless the line is coherent
      const uint64_t* s64 = reinterpret_cast<const uint64_t*>(src + i);
      const uint64_t x = __hip_atomic_load(s64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t y = __hip_atomic_load(s64 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return u32x4{(uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32)};
    } else {
      return src[i];
    }
  };
  size_t i = lo + tid;
  for (; i + (U - 1) * (size_t)nthr < hi; i += U * (size_t)nthr) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld(i + u * (size_t)nthr);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * (size_t)nthr);
  }
  for (; i < hi; i += nthr) __builtin_nontemporal_store(ld(i), dst + i);
}

__global__ __launch_bounds__(kConsumerThreads) void k_consumer(const uint16_t* __restrict__ y,
                                                                BufPtrs bufs, moe_plan_t p,
                                                                const uint32_t* flags,
                                                                uint32_t epoch, uint64_t* trace,
                                                                int trace_seg, int tiles2, int H) {
  __shared__ int s_abort;
  __shared__ __attribute__((aligned(16))) uint32_t s_reserve[kConsumerLdsBytes / 4];
  const int tid = threadIdx.x;
  if (tid == 0) { s_abort = 0; s_reserve[0] = 0; }
  __syncthreads();
  const int n_seg = p.meta[META_NSEG];
  const int nwg = gridDim.x, wg = blockIdx.x;
  const bool tr = trace != nullptr && wg == 0 && tid == 0;
  if (tr) trace[1] = wall_clock64();
  for (int sgi = 0; sgi < n_seg; ++sgi) {
    const int b0 = p.seg_band0[sgi];
    const int nb = p.seg_nbands[sgi];
    if (tr) trace[trace_seg + 3 * sgi] = wall_clock64();
    if (tid < 64) {
      const uint32_t* f = flags + (size_t)b0 * tiles2;
      const int nf = nb * tiles2;
      const uint64_t t_start = wall_clock64();
      while (true) {
        bool ok = true;
        for (int i = tid; i < nf; i += 64)
          ok &= (__hip_atomic_load(f + i, MOE_DEVICE_SCOPE_PUBLISH ? __ATOMIC_RELAXED : __ATOMIC_ACQUIRE,
                                   __HIP_MEMORY_SCOPE_AGENT) == epoch);
        if (__ballot(!ok) == 0ull) break;
        if (wall_clock64() - t_start > kWaitTicks) {
          if (tid == 0) {
            s_abort = 1;
            int expected = 0;
            __hip_atomic_compare_exchange_strong(p.meta + META_STATUS, &expected, MOE_ERR_TIMEOUT,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if (s_abort) return;
    if (!MOE_DEVICE_SCOPE_PUBLISH) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tr) trace[trace_seg + 3 * sgi + 1] = wall_clock64();
    const size_t units = (size_t)p.seg_rows[sgi] * H / 8;
    const size_t per = (units + nwg - 1) / nwg;
    const size_t lo = (size_t)wg * per;
    const size_t hi = lo + per < units ? lo + per : units;
    if (lo < hi) {
      const u32x4* src = reinterpret_cast<const u32x4*>(y + (size_t)p.seg_src_row[sgi] * H);
      u32x4* dst = reinterpret_cast<u32x4*>(bufs.p[p.seg_dest[sgi]] + (size_t)p.seg_dst_row[sgi] * H);
      copy_units<MOE_DEVICE_SCOPE_PUBLISH != 0>(src, dst, lo, hi, tid, kConsumerThreads);
    }
    if (trace != nullptr && wg == 0) {
      __syncthreads();
      if (tid == 0) trace[trace_seg + 3 * sgi + 2] = wall_clock64();
    }
  }
  if (tid == 0 && s_reserve[0] != 0) s_abort = 2;   // keeps the LDS reservation alive
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
    copy_units<false>(src, dst, a, b, threadIdx.x, 256);
  }
}

hipError_t launch_consumer(const Geometry& g, const uint16_t* y, BufPtrs bufs, const moe_plan_t& p,
                           const uint32_t* flags, uint32_t epoch, uint64_t* trace, int n_wg,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_consumer, dim3(n_wg), dim3(kConsumerThreads), 0, st, y, bufs, p, flags,
                     epoch, trace, 8 + g.max_flags, g.tiles2, g.H);
  return hipGetLastError();
}

hipError_t launch_bulk_copy(const Geometry& g, const uint16_t* y, BufPtrs bufs,
                            const moe_plan_t& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_bulk_copy, dim3(grid), dim3(256), 0, st, y, bufs, p, g.H);
  return hipGetLastError();
}

}  // namespace moe
