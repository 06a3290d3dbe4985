// The consumer's copy loop as a device function: the consumer role of the
// overlapped output projection (its first c workgroups) runs it.
//
// Workgroup w of nwg copies the batches of BATCH consecutive 64 KiB copy
// units starting at units (w + i nwg) BATCH, i = 0, 1, ... (the units of all
// segments in schedule order). Before a batch it makes sure that every
// segment up to the batch's last one is ready: wave 0 polls the flags of the
// row tiles of the segments past its own ready frontier, in order
// (consecutive segments mostly share row tiles, which are polled once).
// Workgroups therefore never wait for one another; each keeps ROUND 16-byte
// loads per thread in flight. Flags and rows are read with device-scope
// loads (rows: 16-byte buffer loads with the sc1 policy), which pair with
// the producer's device-scope stores and completion wait; no L2 invalidate
// is issued per segment.
//
// Every wait is bounded: after wait_ticks of the 100 MHz constant clock the
// device status word becomes MOE_ERR_TIMEOUT and the workgroup returns.
#pragma once

#include "common.hpp"

#ifndef MOE_DEVICE_SCOPE_PUBLISH
#define MOE_DEVICE_SCOPE_PUBLISH 1
#endif

namespace moe {

// segment tables staged in LDS: unit0 [kSegLds + 1], then rows, src_row,
// dst_row, dest, tile0, tile1 [kSegLds]; segments past kSegLds are read from
// global memory
constexpr int kSegLds = 2048;
constexpr int kSegLdsBytes = (kSegLds + 1 + 6 * kSegLds) * 4;

struct ConsumerArgs {
  const uint16_t* y;          // expert outputs (published rows)
  BufPtrs bufs;               // combine buffers by owner rank
  const int32_t* meta;        // META_NSEG, META_NUNITS; META_STATUS on timeout
  const int32_t* seg_unit0;
  const int32_t* seg_rows;
  const int32_t* seg_src_row;
  const int32_t* seg_dst_row;
  const int32_t* seg_dest;
  const int32_t* seg_tile0;
  const int32_t* seg_tile1;
  const uint32_t* flags;
  uint32_t epoch;
  uint64_t* trace;            // optional: [1] start, [trace_seg + 3 s + 0/1/2] segment s stamps
  int trace_seg;
  int tiles2;                 // column tiles per row tile (flags per row tile)
  int H;
  uint64_t wait_ticks;        // bound on one wait for a segment's flags (100 MHz ticks)
};

ConsumerArgs consumer_args(const Geometry& g, const uint16_t* y, BufPtrs bufs, const moe_plan_t& p,
                           const uint32_t* flags, uint32_t epoch, uint64_t* trace, uint64_t wait_ticks);

template <int NT, int BATCH, int ROUND>
__device__ void consume(const ConsumerArgs& c, int wg, int nwg, int* s_tab, int* s_abort) {
  constexpr size_t kUnit16 = kCopyUnitBytes / 16;   // 16-byte words per unit
  constexpr int kPer = (int)(kUnit16 / NT);          // words per thread and unit
  constexpr int kSlots = BATCH * kPer;               // words per thread and batch
  static_assert(kUnit16 % NT == 0 && kSlots % ROUND == 0, "rounds split the batch evenly");
  const int tid = threadIdx.x;
  const int n_seg = c.meta[META_NSEG];
  const int n_units = c.meta[META_NUNITS];
  const int H = c.H;
  int* t_unit0 = s_tab;
  int* t_rows = s_tab + kSegLds + 1;
  int* t_src = t_rows + kSegLds;
  int* t_dst = t_src + kSegLds;
  int* t_dest = t_dst + kSegLds;
  int* t_t0 = t_dest + kSegLds;
  int* t_t1 = t_t0 + kSegLds;
  const int n_lds = min(n_seg, kSegLds);
  for (int i = tid; i < n_lds; i += NT) {
    t_unit0[i] = c.seg_unit0[i];
    t_rows[i] = c.seg_rows[i];
    t_src[i] = c.seg_src_row[i];
    t_dst[i] = c.seg_dst_row[i];
    t_dest[i] = c.seg_dest[i];
    t_t0[i] = c.seg_tile0[i];
    t_t1[i] = c.seg_tile1[i];
  }
  if (tid == 0) {
    t_unit0[n_lds] = n_lds < n_seg ? c.seg_unit0[n_lds] : n_units;
    *s_abort = 0;
  }
  __syncthreads();
  auto unit0 = [&](int i) {
    if (i <= n_lds) return t_unit0[i];
    return i < n_seg ? c.seg_unit0[i] : n_units;
  };
  auto field = [&](const int* lds, const int32_t* glob, int i) { return i < n_lds ? lds[i] : glob[i]; };
  const bool tr = c.trace != nullptr && wg == 0 && tid == 0;
  if (tr) c.trace[1] = wall_clock64();
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
        const int t0 = field(t_t0, c.seg_tile0, ready), t1 = field(t_t1, c.seg_tile1, ready);
        if (t0 >= kt0 && t1 <= kt1) continue;
        const uint32_t* f = c.flags + (size_t)t0 * c.tiles2;
        const int nf = (t1 - t0 + 1) * c.tiles2;
        const uint64_t t_start = wall_clock64();
        if (tr) c.trace[c.trace_seg + 3 * ready] = t_start;
        bool timed_out = false;
        while (true) {
          bool ok = true;
          for (int i = tid; i < nf; i += 64)
            ok &= (__hip_atomic_load(f + i, MOE_DEVICE_SCOPE_PUBLISH ? __ATOMIC_RELAXED : __ATOMIC_ACQUIRE,
                                     __HIP_MEMORY_SCOPE_AGENT) == c.epoch);
          if (__ballot(!ok) == 0ull) break;
          if (wall_clock64() - t_start > c.wait_ticks) { timed_out = true; break; }
          __builtin_amdgcn_s_sleep(2);
        }
        if (timed_out) {
          if (tid == 0) {
            *s_abort = 1;
            int expected = 0;
            __hip_atomic_compare_exchange_strong(const_cast<int32_t*>(c.meta) + META_STATUS, &expected,
                                                 MOE_ERR_TIMEOUT, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          break;
        }
        kt0 = t0;
        kt1 = t1;
        if (tr) c.trace[c.trace_seg + 3 * ready + 1] = wall_clock64();
      }
    }
    __syncthreads();
    if (*s_abort) return;
    if (!MOE_DEVICE_SCOPE_PUBLISH) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the batch's units: a buffer resource over each unit's source bytes (a
    // missing unit has none: its loads return zeros and nothing is stored)
    __amdgpu_buffer_rsrc_t src[BATCH];
    u32x4* dst[BATCH];
    uint32_t n16[BATCH];   // 16-byte words of the unit
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = u0 + k;
      const uint16_t* sp = c.y;
      dst[k] = reinterpret_cast<u32x4*>(c.bufs.p[0]);
      n16[k] = 0;
      if (u < u1) {
        while (seg + 1 < n_seg && unit0(seg + 1) <= u) ++seg;
        const uint32_t words = (uint32_t)field(t_rows, c.seg_rows, seg) * (uint32_t)(H / 8);
        const uint32_t lo = (uint32_t)(u - unit0(seg)) * (uint32_t)kUnit16;
        n16[k] = lo + (uint32_t)kUnit16 < words ? (uint32_t)kUnit16 : words - lo;
        sp = c.y + (size_t)field(t_src, c.seg_src_row, seg) * H + (size_t)lo * 8;
        dst[k] = reinterpret_cast<u32x4*>(c.bufs.p[field(t_dest, c.seg_dest, seg)] +
                                          (size_t)field(t_dst, c.seg_dst_row, seg) * H) + lo;
      }
      src[k] = buf_rsrc(sp, n16[k] * 16u);
    }
    // rounds of ROUND loads per thread, all in flight before the stores;
    // only the stores are predicated
#pragma unroll
    for (int z0 = 0; z0 < kSlots; z0 += ROUND) {
      u32x4 v[ROUND];
#pragma unroll
      for (int z = 0; z < ROUND; ++z) {
        const int k = (z0 + z) / kPer, q = (z0 + z) % kPer;
        const uint32_t i = (uint32_t)(q * NT + tid);
        v[z] = __builtin_amdgcn_raw_buffer_load_b128(src[k], i * 16u, 0,
                                                     MOE_DEVICE_SCOPE_PUBLISH ? kCpolDevice : 0);
      }
#pragma unroll
      for (int z = 0; z < ROUND; ++z) {
        const int k = (z0 + z) / kPer, q = (z0 + z) % kPer;
        const uint32_t i = (uint32_t)(q * NT + tid);
        if (i < n16[k]) store16_nt(dst[k] + i, v[z]);
      }
    }
    if (c.trace != nullptr && wg == 0) {
      __syncthreads();
      if (tid == 0) c.trace[c.trace_seg + 3 * last + 2] = wall_clock64();
    }
  }
}

}  // namespace moe
