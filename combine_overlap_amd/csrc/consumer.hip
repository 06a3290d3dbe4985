// Consumer of the tile-signalling overlap paper (sec. 3.3.2-3.3.3): a
// persistent kernel on a small set of CUs that walks the transfer segments
// in schedule order, waits until every tile of a segment's row bands carries
// the current epoch flag (acquire loads at agent scope), and then moves the
// segment's valid rows with one contiguous copy into the combine buffer of
// the owner rank. Flags and rows are read with device-scope loads, which
// pair with the producer's device-scope stores and completion wait (see the
// output-projection epilogue); no L2 invalidate is issued per segment. On
// one GPU the owner's receive buffer is a buffer in local HBM. The segments'
// rows are cut into 64 KiB copy units, dealt to the c consumer workgroups in
// batches (see k_consumer).
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
constexpr int kConsumerThreads = 1024;   // CU-partition consumer
constexpr int kConsumerLdsBytes = 80 * 1024;
// segment tables staged in the consumer's LDS (the reservation has room):
// unit0 [kSegLds + 1], then rows, src_row, dst_row, dest, tile0, tile1 [kSegLds]
constexpr int kSegLds = 2048;
static_assert((kSegLds + 1 + 6 * kSegLds) * 4 <= kConsumerLdsBytes, "segment tables fit the reservation");

#ifndef MOE_DEVICE_SCOPE_PUBLISH
#define MOE_DEVICE_SCOPE_PUBLISH 1
#endif

// 64 KiB copy units per consumer batch (loads in flight per workgroup)
#ifndef MOE_CONSUMER_BATCH
#define MOE_CONSUMER_BATCH 4
#endif
constexpr int kBatchUnits = MOE_CONSUMER_BATCH;

#ifndef MOE_COPY_UNROLL
#define MOE_COPY_UNROLL 8
#endif

template <bool DEVICE_SCOPE>
__device__ __forceinline__ u32x4 load16(const u32x4* a) {
  if constexpr (DEVICE_SCOPE) return load16_device(a);
  else return *(const GLOBAL_AS u32x4*)a;
}

// plain 16-byte loads (non-temporal loads halve the per-CU rate), streaming
// stores; MOE_COPY_UNROLL loads in flight per thread
__device__ __forceinline__ void copy_units(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                           size_t lo, size_t hi, int tid, int nthr) {
  constexpr int U = MOE_COPY_UNROLL;
  size_t i = lo + tid;
  for (; i + (U - 1) * (size_t)nthr < hi; i += U * (size_t)nthr) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * (size_t)nthr];
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * (size_t)nthr);
  }
  for (; i < hi; i += nthr) __builtin_nontemporal_store(src[i], dst + i);
}

// Workgroup w copies the batches of BATCH consecutive 64 KiB copy units
// starting at units (w + i c) BATCH, i = 0, 1, ... (the units of all segments
// in schedule order). Before a batch it makes sure that every segment up to
// the batch's last one is ready: wave 0 polls the flags of the row tiles of
// the segments past its own ready frontier, in order (consecutive segments
// mostly share row tiles, which are polled once). Workgroups therefore never
// wait for one another; each keeps ROUND 16-byte loads per thread in flight.
//
// One workgroup of NT threads per consumer CU; the segment tables are staged
// in an LDS reservation large enough that no producer workgroup shares the CU.
template <int NT, int BATCH, int ROUND, bool LDS_TABLES>
__global__ __launch_bounds__(NT) void k_consumer(const uint16_t* __restrict__ y,
                                                                    BufPtrs bufs, moe_plan_t p,
                                                                    const uint32_t* flags,
                                                                    uint32_t epoch, uint64_t* trace,
                                                                    int trace_seg, int tiles2, int H) {
  constexpr size_t kUnit16 = kCopyUnitBytes / 16;                 // 16-byte words per unit
  constexpr int kPer = (int)(kUnit16 / NT);                        // words per thread and unit
  constexpr int kSlots = BATCH * kPer;                             // words per thread and batch
  static_assert(kSlots % ROUND == 0, "rounds split the batch evenly");
  __shared__ int s_abort;
  __shared__ __attribute__((aligned(16))) int s_tab[LDS_TABLES ? kConsumerLdsBytes / 4 : 1];
  const int tid = threadIdx.x;
  const int n_seg = p.meta[META_NSEG];
  const int n_units = p.meta[META_NUNITS];
  // segment tables: the first kSegLds segments from LDS, any others from global memory
  int* t_unit0 = s_tab;
  int* t_rows = s_tab + kSegLds + 1;
  int* t_src = t_rows + kSegLds;
  int* t_dst = t_src + kSegLds;
  int* t_dest = t_dst + kSegLds;
  int* t_t0 = t_dest + kSegLds;
  int* t_t1 = t_t0 + kSegLds;
  const int n_lds = LDS_TABLES ? min(n_seg, kSegLds) : 0;
  if constexpr (LDS_TABLES) {
    for (int i = tid; i < n_lds; i += NT) {
      t_unit0[i] = p.seg_unit0[i];
      t_rows[i] = p.seg_rows[i];
      t_src[i] = p.seg_src_row[i];
      t_dst[i] = p.seg_dst_row[i];
      t_dest[i] = p.seg_dest[i];
      t_t0[i] = p.seg_tile0[i];
      t_t1[i] = p.seg_tile1[i];
    }
    if (tid == 0) t_unit0[n_lds] = n_lds < n_seg ? p.seg_unit0[n_lds] : n_units;
  }
  if (tid == 0) s_abort = 0;
  __syncthreads();
  auto unit0 = [&](int i) {
    if (LDS_TABLES && i <= n_lds) return t_unit0[i];
    return i < n_seg ? p.seg_unit0[i] : n_units;
  };
  auto field = [&](const int* lds, const int32_t* glob, int i) {
    return (LDS_TABLES && i < n_lds) ? lds[i] : glob[i];
  };
  const int nwg = gridDim.x, wg = blockIdx.x;
  const bool tr = trace != nullptr && wg == 0 && tid == 0;
  if (tr) trace[1] = wall_clock64();
  int ready = 0;             // wave 0: segments [0, ready) are known to be ready
  int kt0 = 1, kt1 = 0;      // wave 0: row tiles [kt0, kt1] seen flagged (empty at first)
  int seg = 0;               // segment of the unit being placed (non-decreasing)
  for (int u0 = wg * BATCH; u0 < n_units; u0 += nwg * BATCH) {
    const int u1 = min(u0 + BATCH, n_units);
    int last = seg;    // segment of unit u1 - 1
    while (last + 1 < n_seg && unit0(last + 1) <= u1 - 1) ++last;
    if (tid < 64) {
      for (; ready <= last; ++ready) {
        // every column tile of the row tiles covering the segment's bands
        const int t0 = field(t_t0, p.seg_tile0, ready), t1 = field(t_t1, p.seg_tile1, ready);
        if (t0 >= kt0 && t1 <= kt1) continue;
        const uint32_t* f = flags + (size_t)t0 * tiles2;
        const int nf = (t1 - t0 + 1) * tiles2;
        const uint64_t t_start = wall_clock64();
        if (tr) trace[trace_seg + 3 * ready] = t_start;
        bool timed_out = false;
        while (true) {
          bool ok = true;
          for (int i = tid; i < nf; i += 64)
            ok &= (__hip_atomic_load(f + i, MOE_DEVICE_SCOPE_PUBLISH ? __ATOMIC_RELAXED : __ATOMIC_ACQUIRE,
                                     __HIP_MEMORY_SCOPE_AGENT) == epoch);
          if (__ballot(!ok) == 0ull) break;
          if (wall_clock64() - t_start > kWaitTicks) { timed_out = true; break; }
          __builtin_amdgcn_s_sleep(2);
        }
        if (timed_out) {
          if (tid == 0) {
            s_abort = 1;
            int expected = 0;
            __hip_atomic_compare_exchange_strong(p.meta + META_STATUS, &expected, MOE_ERR_TIMEOUT,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          break;
        }
        kt0 = t0;
        kt1 = t1;
        if (tr) trace[trace_seg + 3 * ready + 1] = wall_clock64();
      }
    }
    __syncthreads();
    if (s_abort) return;
    if (!MOE_DEVICE_SCOPE_PUBLISH) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the batch's units (a missing unit reads row 0 of y and stores nothing)
    const u32x4* src[BATCH];
    u32x4* dst[BATCH];
    uint32_t lo[BATCH], hi[BATCH], last_ld[BATCH];   // 16-byte words in the segment
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = u0 + k;
      src[k] = reinterpret_cast<const u32x4*>(y);
      dst[k] = reinterpret_cast<u32x4*>(bufs.p[0]);
      lo[k] = 0;
      hi[k] = 0;
      last_ld[k] = 0;
      if (u < u1) {
        while (seg + 1 < n_seg && unit0(seg + 1) <= u) ++seg;
        const uint32_t words = (uint32_t)field(t_rows, p.seg_rows, seg) * (uint32_t)(H / 8);
        lo[k] = (uint32_t)(u - unit0(seg)) * (uint32_t)kUnit16;
        hi[k] = lo[k] + (uint32_t)kUnit16 < words ? lo[k] + (uint32_t)kUnit16 : words;
        last_ld[k] = hi[k] - 1;
        src[k] = reinterpret_cast<const u32x4*>(y + (size_t)field(t_src, p.seg_src_row, seg) * H);
        dst[k] = reinterpret_cast<u32x4*>(bufs.p[field(t_dest, p.seg_dest, seg)] +
                                          (size_t)field(t_dst, p.seg_dst_row, seg) * H);
      }
    }
    // rounds of ROUND loads per thread: the loads are unconditional (indices
    // clamped into the unit) so the compiler keeps them all in flight; only
    // the stores are predicated
#pragma unroll
    for (int z0 = 0; z0 < kSlots; z0 += ROUND) {
      u32x4 v[ROUND];
#pragma unroll
      for (int z = 0; z < ROUND; ++z) {
        const int k = (z0 + z) / kPer, q = (z0 + z) % kPer;
        const uint32_t i = lo[k] + (uint32_t)(q * NT + tid);
        v[z] = load16<MOE_DEVICE_SCOPE_PUBLISH != 0>(src[k] + (i < last_ld[k] ? i : last_ld[k]));
      }
#pragma unroll
      for (int z = 0; z < ROUND; ++z) {
        const int k = (z0 + z) / kPer, q = (z0 + z) % kPer;
        const uint32_t i = lo[k] + (uint32_t)(q * NT + tid);
        if (i < hi[k]) store16_nt(dst[k] + i, v[z]);
      }
    }
    if (trace != nullptr && wg == 0) {
      __syncthreads();
      if (tid == 0) trace[trace_seg + 3 * last + 2] = wall_clock64();
    }
  }
  if constexpr (LDS_TABLES)   // keeps the whole reservation
    if (tid == 0 && s_tab[kConsumerLdsBytes / 4 - 1] == 0x7fffffff) s_abort = 2;
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

hipError_t launch_consumer(const Geometry& g, const uint16_t* y, BufPtrs bufs, const moe_plan_t& p,
                           const uint32_t* flags, uint32_t epoch, uint64_t* trace, int n_wg,
                           hipStream_t st) {
  hipLaunchKernelGGL((k_consumer<kConsumerThreads, kBatchUnits, 16, true>), dim3(n_wg),
                     dim3(kConsumerThreads), 0, st, y, bufs, p, flags, epoch, trace, 8 + g.max_flags,
                     g.tiles2, g.H);
  return hipGetLastError();
}

hipError_t launch_bulk_copy(const Geometry& g, const uint16_t* y, BufPtrs bufs,
                            const moe_plan_t& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_bulk_copy, dim3(grid), dim3(256), 0, st, y, bufs, p, g.H);
  return hipGetLastError();
}

}  // namespace moe
