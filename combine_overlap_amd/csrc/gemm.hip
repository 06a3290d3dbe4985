// Producer: the rank-wide persistent grouped GEMM of the tile-signalling
// overlap paper (sec. 3.3.1). One launch covers every local expert through
// one tile worklist: tile t = (row tile at schedule position t / tiles_n,
// column tile t % tiles_n), row tiles in the remote-first schedule order
// (sec. 3.2.2). The expert of a row tile selects the weight pointer; no
// matrices are concatenated and nothing is relaunched per expert.
//
// Row tiles are 256 rows of one expert's tb_m-aligned rows, whatever the
// band height tb_m (the padding and transfer unit of the row layout): the
// last tile of an expert is shorter and stores only its own rows (the rows
// past them, read from the next expert or the buffer's slack, are computed
// and discarded). The paper ties the tile to the band; here a small band
// keeps the owner-group padding small while the tile stays at the size that
// runs the MFMA pipes best.
//
// gfx950 mapping
//  * Tile queues per XCD: each XCD's L2 sees a fixed subset of column tiles
//    (weight slices) and of row tiles, in schedule order. A workgroup reads its XCD from HW_REG_XCC_ID and takes the next
//    tile of that XCD's queue with one atomic; when the queue is empty it
//    steals from the other queues. Any grid size and any placement of the
//    consumer's CUs therefore keeps every producer CU busy.
//  * Split tail: an XCD queue of T tiles served by P workgroups runs T / P
//    full rounds; its last T mod P tiles would leave most of that XCD idle
//    for a whole tile time, so each of them is cut into s = P / (T mod P)
//    chunks along K (at most 4 in the first projection, 8 in the output
//    projection). A chunk stores its fp32 accumulators as a partial tile
//    (device-scope write-through stores), waits for them to complete and
//    increments the tile's arrival counter. First projection: the chunk that
//    arrives last adds the other partials and runs the epilogue. Output
//    projection: every chunk waits (bounded) for all partials, adds the
//    partials of its share of the accumulator blocks and stores it; the last
//    chunk to store raises the tile's flag. Partials are always added in
//    chunk order, so the bits do not depend on the arrival order.
//  * CU partition (optional, output projection): the launch's first c
//    workgroups run the consumer (consumer.hpp) first; once their share of
//    the copy is done they take tiles like the others.
//  * Gathered rows (optional, first projection): A row r of a tile is row
//    row_src[r] of x, loaded through a buffer resource over x with 32-bit
//    offsets; padding rows sit at an offset past the resource's end and land
//    zeros. An x of 2 GiB or more uses per-lane 64-bit addresses and a zero
//    row instead.
//  * Short tiles: the 32-row blocks past an expert's last row skip their
//    MFMAs, and their DMA re-reads the tile's first rows (L2 hits).
//  * Role switching (optional, output projection): the workgroups also do
//    the consumer's work. Before each tile a workgroup claims the next eight
//    64 KiB copy units (one fetch-and-add) if the segment holding them has
//    all its row tiles flagged and copies them into their owner's combine
//    buffer, repeating while units are ready; once the tiles run out the
//    workgroups claim, wait for and copy the rest. The copy thus takes the
//    CU-microseconds it costs instead of a standing partition of CUs.
//  * 4 or 8 waves per workgroup in a WM x WN grid (8 = two waves per SIMD);
//    v_mfma_f32_16x16x32_bf16 with fp32 accumulators (four per 32x32 block).
//  * The k-loop streams BK-wide slices of A and B straight from global memory
//    into an NS-stage LDS ring with global_load_lds_dwordx4 (no VGPR staging).
//    Each lane fetches the 16-byte chunk that belongs at its LDS slot under an
//    XOR swizzle that keeps MFMA fragment reads free of bank conflicts. One
//    barrier per k-step: wait for this wave's copies of stage kt, barrier,
//    issue stage kt+NS-1 into the slot freed by stage kt-1 in two halves
//    around the step's last MFMAs, run the MFMAs.
//
// Epilogues:
//   EPI_PLAIN  C = A B^T (output projection y = h W2^T). With flags the tile
//              is published as in sec. 3.3.1 (store, fence, flag): its rows go
//              out with device-scope (sc1) stores, which write through this
//              XCD's L2 to the device coherence point; s_waitcnt vmcnt(0)
//              waits until every one of them has completed; the workgroup
//              synchronises; one lane stores flags[t] = epoch (device scope).
//              The consumer polls with device-scope loads and reads the rows
//              with device-scope loads, so it sees the completed stores. This
//              is the ordering an agent-scope release/acquire pair provides,
//              without the whole-L2 writeback (producer) and invalidate
//              (consumer) those need for ordinary cached accesses, which cost
//              ~15% of the producer's time when issued once per tile.
//              (Build with -DMOE_DEVICE_SCOPE_PUBLISH=0 for the fence-based
//              release/acquire form.)
//   EPI_SILU   h = SiLU(x W1^T)                        (non-gated FFN)
//   EPI_GATED  h = SiLU(x W1^T) * (x W3^T); the B tile interleaves 32-row
//              blocks of W1 and W3 so each wave holds u and v of the same h
//              columns in registers.
#include <type_traits>

#include "consumer.hpp"

#ifndef MOE_DEVICE_SCOPE_PUBLISH
#define MOE_DEVICE_SCOPE_PUBLISH 1
#endif

namespace moe {

enum { EPI_PLAIN = 0, EPI_SILU = 1, EPI_GATED = 2 };

#define LDS_AS __attribute__((address_space(3)))

// K chunks per split tail tile. In the first projection the last chunk to
// arrive reduces the whole tile, so few chunks pay; in the output projection
// every chunk reduces and stores its own share of the tile's accumulator
// blocks, so up to one chunk per block.
constexpr int kMaxSplitSerial = 4;
constexpr int kMaxSplitShared = 8;
constexpr int kMinSplitSteps = 8;   // k-steps per chunk at least
// ... and in the output projection when a queue holds less than one round of
// tiles (a launch-bound layer: H = 512, F = 1024 gives 6 tiles of 16 k-steps
// for 256 workgroups), where the chunks share the reduction: its output
// projection 38 -> 30 us on MI355X. Not in the first projection, whose last
// chunk sums the whole tile alone (there 4-step chunks were slower: 28 ->
// 35 us), nor past one round, where the split only evens out the last one.
constexpr int kMinSplitStepsSparse = 4;
// buffer offset of gathered padding rows: past any x a resource describes
// (x must stay below 2 GiB for the buffer form, so offset + k offset < 2^32)
constexpr uint32_t kBufOutOfRange = 0x80000000u;
// split tail tiles per XCD queue at most (tail * nsplit <= kTailSlots with
// nsplit >= 2): word 1 + t of the queue's counter block counts tile t's
// chunk arrivals and stored shares, word 1 + kTailTiles + t its claimed shares
constexpr int kTailTiles = kTailSlots / 2;
static_assert(1 + 2 * kTailTiles <= kCtrStride, "tail words fit the counter block");


template <int BM, int BN, int BK, int NS, int WM, int WN>
struct Tile {
  static constexpr int NW = WM * WN;                   // waves per workgroup (4 or 8)
  static constexpr int NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int CPR = BK / 8;          // 16-byte chunks per LDS row
  static constexpr int RPI = 64 / CPR;        // rows covered by one wave-wide DMA instruction
  static constexpr int A_PW = BM / RPI / NW;  // DMA instructions per wave per stage (A)
  static constexpr int B_PW = BN / RPI / NW;  // (B)
  static constexpr int LPW = A_PW + B_PW;
  static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
  static constexpr int RING = NS * STAGE;
  static constexpr int EPI_ROW = BN + 8;        // padded LDS row of the staged output tile
  static constexpr int LDS_ELEMS = RING > BM * EPI_ROW ? RING : BM * EPI_ROW;
  static_assert((NW == 4 || NW == 8) && FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0,
                "wave tiling");
  static_assert(A_PW >= 1 && B_PW >= 1 && (BM / RPI) % NW == 0 && (BN / RPI) % NW == 0, "dma split");
  static_assert(NS >= 2 && (NS - 1) * LPW <= 63, "vmcnt range");
  static_assert(BK % 32 == 0, "even number of k16 substeps per stage");
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS");
};

struct GemmArgs {
  const uint16_t* A;           // [rows, K]; gathered: [a_nrows, K] rows picked by a_rows
  const int32_t* a_rows;       // gathered first projection: source row of each packed row
                               // (-1 = padding), rows >= meta[META_MPAD] read as padding
  const uint16_t* a_zero;      // [K] zeros: the source of padding rows
  int a_nrows;
  const uint16_t* B0;          // [El, Nw, K]
  const uint16_t* B1;          // [El, Nw, K] (gated only)
  uint16_t* C;                 // [rows, Nout]
  const int32_t* meta;
  const int32_t* tile_row0;    // row tiles in layout order: first row, expert, rows
  const int32_t* tile_expert;
  const int32_t* tile_rows;
  const int32_t* tile_sched;   // schedule position -> row tile
  int32_t* my_ctr;             // this launch's 8 per-XCD queue counters
  int32_t* other_ctr;          // the other launch's counters (zeroed here)
  float* partial;              // fp32 partial tiles of split tail tiles, [8 * kTailSlots][BM * BN]
  uint32_t* flags;             // output projection: the ready flags it raises (null: none);
                               // first projection: the flags it clears for the output projection
  // role switching (output projection): the consumer's copy duty between tiles
  int copy_duty;
  int32_t* my_copy;            // copy duty: [0] next unclaimed copy unit, [1] segment search hint
  int32_t* other_copy;         // the other launch's copy words (cleared here)
  BufPtrs bufs;                // combine buffers by source rank
  const int32_t* seg_tile0;
  const int32_t* seg_tile1;
  const int32_t* seg_unit0;    // first 64 KiB copy unit of each segment
  const int32_t* seg_rows;
  const int32_t* seg_src_row;
  const int32_t* seg_dst_row;
  const int32_t* seg_dest;
  int flags_n;                 // first projection: flags per row tile of the output projection
  uint64_t* trace;             // optional timeline: [0] start, [8 + t] tile t done
  // CU-partition overlap inside one launch: workgroups [0, n_cons) run the
  // consumer (one per CU, n_cons / 8 per XCD), the others the tiles;
  // -1: the plan's choice meta[META_CAUTO]
  int n_cons;
  ConsumerArgs cons;
  uint32_t epoch;
  uint64_t wait_ticks;         // bound on one wait of the copy duty for a segment's flags
  int K, Nw, Nout, tiles_n;
  int xb, xn;                  // XCD grid: xcd = (row tile % xb) * xn + (column tile % xn)
  int gp, gq;                  // blocks of gp row tiles x gq column tiles inside an XCD queue
  int px;                      // workgroups per XCD queue the tail split is sized for;
                               // 0: (grid - meta[META_CAUTO]) / 8
  uint64_t tail_wait_ticks;    // output projection: bound on a split tail chunk's wait for
                               // its tile's other chunks (then the last to arrive takes its share)
  // test knobs (timing only; the results do not change): a nonzero seed
  // delays each work item by a seeded number of sleeps before its stores;
  // reverse walks every queue's whole tiles in reverse schedule order
  uint32_t dbg_seed;
  int dbg_reverse;
};

// Queue index i of XCD x -> tile (row-tile schedule position * tiles_n + column tile).
// XCD x owns row tiles b = bx + k*xb and column tiles t = nx + l*xn; its queue walks
// blocks of gp row tiles x gq column tiles (in schedule order, so remote rows
// still finish first) so that the tiles an XCD runs at about the same time
// share A rows and weight columns in its L2. The row tiles holding a remote band (the first
// n_rrt schedule positions) and the others are blocked separately, so no block
// mixes them: the last tiles to finish are then local ones where there are
// enough, and the copy of the remote rows need not wait for the launch's last
// round. Returns -1 past the end of the queue.
__device__ __forceinline__ int queue_tile(const GemmArgs& a, int n_rt, int n_rrt, int x, int i) {
  const int bx = x / a.xn, nx = x - (x / a.xn) * a.xn;
  if (bx >= n_rt || nx >= a.tiles_n) return -1;
  const int nb = (n_rt - bx + a.xb - 1) / a.xb;         // row tiles of this XCD
  const int nn = (a.tiles_n - nx + a.xn - 1) / a.xn;    // column tiles of this XCD
  if (i >= nb * nn) return -1;
  // row tiles k < kr of this XCD hold a remote band
  const int kr = min(nb, max(0, (n_rrt - bx + a.xb - 1) / a.xb));
  int k0 = 0, nk = kr;
  if (i >= kr * nn) {
    i -= kr * nn;
    k0 = kr;
    nk = nb - kr;
  }
  const int per_group = a.gp * nn;
  const int g = i / per_group;
  const int pg = min(a.gp, nk - g * a.gp);              // row tiles in this group
  const int rem = i - g * per_group;
  const int h = rem / (pg * a.gq);
  const int qh = min(a.gq, nn - h * a.gq);              // column tiles in this block
  const int rem2 = rem - h * pg * a.gq;
  const int k = k0 + g * a.gp + rem2 / qh;
  const int l = h * a.gq + rem2 % qh;
  return (bx + k * a.xb) * a.tiles_n + (nx + l * a.xn);
}

// Work item i of XCD queue x, served by px workgroups: the first T - tail
// items are whole tiles in queue order; the tail's tiles are split into
// nsplit consecutive K chunks. tail * nsplit <= px: a chunk that waits for
// its tile's other chunks never waits for an item no workgroup is free to
// take (the chunks of all queues together are at most the producer's
// workgroups, and a workgroup holds one chunk at a time). slot = index among the split items (< kTailSlots),
// slot / nsplit = the tail tile's arrival counter.
struct Item {
  int tile, chunk, nsplit, slot;
};

__device__ __forceinline__ Item queue_item(const GemmArgs& a, int n_rt, int n_rrt, int x, int i, int px, int nk,
                                           int max_split, int min_steps_sparse) {
  Item it{-1, 0, 1, 0};
  const int bx = x / a.xn, nx = x - (x / a.xn) * a.xn;
  if (bx >= n_rt || nx >= a.tiles_n) return it;
  const int nb = (n_rt - bx + a.xb - 1) / a.xb;
  const int nn = (a.tiles_n - nx + a.xn - 1) / a.xn;
  const int T = nb * nn;
  const int tail = T % px;
  int s = tail > 0 ? px / tail : 1;
  s = min(s, min(max_split, nk / (T < px ? min_steps_sparse : kMinSplitSteps)));
  if (tail * s > kTailSlots) s = kTailSlots / tail;
  // test knob: the whole tiles in reverse queue order (the split tail tiles
  // stay the same tiles, so every tile is summed as without the knob)
  if (s < 2) {
    if (i < T) it.tile = queue_tile(a, n_rt, n_rrt, x, a.dbg_reverse ? T - 1 - i : i);
    return it;
  }
  const int full = T - tail;
  if (i < full) {
    it.tile = queue_tile(a, n_rt, n_rrt, x, a.dbg_reverse ? full - 1 - i : i);
    return it;
  }
  const int j = i - full;
  if (j >= tail * s) return it;
  it.tile = queue_tile(a, n_rt, n_rrt, x, full + j / s);
  it.chunk = j % s;
  it.nsplit = s;
  it.slot = j;
  return it;
}

// physical 16-byte chunk of logical chunk c in LDS row r
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 8) return c ^ (r & 7) ^ ((r >> 3) & 1);
  else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}

__device__ __forceinline__ float silu_f32(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  // lgkmcnt(0): this wave's LDS reads of the slot about to be refilled have completed
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One wave-wide 16-byte-per-lane copy global -> LDS: lane l reads gbase +
// lane_off (gbase wave-uniform, in SGPRs) and lands at lds_byte + 16 l.
// Issued through asm so the compiler does not add a full vmcnt wait before every
// later LDS read; the k-loop waits for exactly the stage it consumes instead.
// The instruction has no VGPR result (the inline-asm load hazard does not apply).
__device__ __forceinline__ void dma16(const void* gbase, uint32_t lane_off, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_off), "s"(gbase), "s"(lds_byte)
      : "memory");
}

// The same copy with a per-lane 64-bit address (rows gathered from anywhere).
__device__ __forceinline__ void dma16_v(const void* lane_addr, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_addr), "s"(lds_byte)
      : "memory");
}

// The same copy through a buffer resource (base, byte size) with a per-lane
// 32-bit offset: a lane whose offset is at or past the resource's size lands
// zeros in the LDS without touching memory.
typedef int moe_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16_buf(uint32_t lane_off, moe_i32x4 rsrc, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_off), "s"(rsrc), "s"(lds_byte)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const LDS_AS void*)p));
}

__device__ __forceinline__ int xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & (kXcds - 1);
}


// Copies 16-byte words [w0, w1) of remote segment sg's valid rows (y rows
// published by other workgroups) into its owner's combine buffer with all NT
// threads: rounds of kRound device-scope 16-byte loads per thread through a
// buffer resource over those words (loads past its end return zeros and are
// not stored; a segment is below 2 GiB, which the host checks).
template <int NT>
__device__ __forceinline__ void copy_words(const GemmArgs& a, int sg, uint32_t w0, uint32_t w1, int tid) {
  constexpr int kRound = 32;   // 16-byte loads per thread in flight
  const int H = a.Nout;
  const uint32_t words = w1 - w0;
  const uint16_t* src = a.C + (size_t)a.seg_src_row[sg] * H + (size_t)w0 * 8;
  u32x4* dst = reinterpret_cast<u32x4*>(a.bufs.p[a.seg_dest[sg]] + (size_t)a.seg_dst_row[sg] * H) + w0;
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(src, words * 16u);
  for (uint32_t i0 = 0; i0 < words; i0 += NT * kRound) {
    u32x4 v[kRound];
#pragma unroll
    for (int z = 0; z < kRound; ++z)
      v[z] = __builtin_amdgcn_raw_buffer_load_b128(r, (i0 + (uint32_t)(z * NT + tid)) * 16u, 0,
                                                   MOE_DEVICE_SCOPE_PUBLISH ? kCpolDevice : 0);
#pragma unroll
    for (int z = 0; z < kRound; ++z) {
      const uint32_t i = i0 + (uint32_t)(z * NT + tid);
      if (i < words) store16_nt(dst + i, v[z]);
    }
  }
}

// device clock stamps of an overlapped output projection (100 MHz ticks),
// cleared by the first projection: META_T_PROD the latest completion of a
// tile, META_T_CONS the latest completion of a copy (consumer workgroups of
// the CU partition, the copy duty of role switching)
__device__ __forceinline__ void stamp_max(const int32_t* meta, int word) {
  uint64_t* w = reinterpret_cast<uint64_t*>(const_cast<int32_t*>(meta) + word);
  __hip_atomic_fetch_max(w, (uint64_t)wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The copy duty, in the 64 KiB copy units of the remote segments (schedule
// order). Word 0 of the copy words is the next unclaimed unit; units are
// claimed kClaimUnits at a time by fetch-and-add, so claiming never retries
// and a large segment is copied by several workgroups. A claim stays with
// its workgroup (s_copy[3..4]) until copied, one segment piece at a time.
//  wait = false (between tiles): copy the pieces of the workgroup's claim
//    whose segments have all their row tiles flagged; with no claim left,
//    claim the next units if the segment holding the first unclaimed unit
//    is ready. Return at the first piece that is not ready.
//  wait = true (no tiles left): the same, but wait (bounded) for each
//    piece's flags; return once every unit is taken and copied.
// Word 1 is a segment search hint: the largest segment found so far.
constexpr int kClaimUnits = 8;

template <int NT>
__device__ void copy_duty(const GemmArgs& a, bool wait, int tid, int* s_copy) {
  const int n_seg = a.meta[META_NSEG];
  const int n_units = a.meta[META_NUNITS];
  const int lane = tid & 63;
  int32_t* next_unit = a.my_copy;
  int32_t* seg_hint = a.my_copy + 1;
  auto tiles_ready = [&](int sg) {
    const int t0 = a.seg_tile0[sg], t1 = a.seg_tile1[sg];
    const int nf = (t1 - t0 + 1) * a.tiles_n;
    const uint32_t* f = a.flags + (size_t)t0 * a.tiles_n;
    bool ok = true;
    for (int i = lane; i < nf; i += 64)
      ok &= (__hip_atomic_load(f + i, MOE_DEVICE_SCOPE_PUBLISH ? __ATOMIC_RELAXED : __ATOMIC_ACQUIRE,
                               __HIP_MEMORY_SCOPE_AGENT) == a.epoch);
    return __ballot(!ok) == 0ull;
  };
  auto unit_end = [&](int sg) { return sg + 1 < n_seg ? a.seg_unit0[sg + 1] : n_units; };
  // wave 0: the segment holding unit u < n_units, i.e. the last one starting
  // at or below u (segment starts are non-decreasing), searched 64 segments
  // at a time from `from`, a segment starting at or below u. The shared hint
  // is used instead when it too starts at or below u.
  auto find_seg = [&](int u, int from) {
    const int h = __hip_atomic_load(seg_hint, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int s0 = (h > from && a.seg_unit0[h] <= u) ? h : from;
    while (true) {
      const int sc = s0 + 1 + lane;
      const int cnt = __popcll(__ballot(sc < n_seg && a.seg_unit0[sc] <= u));
      s0 += cnt;
      if (cnt < 64) break;
    }
    if (lane == 0 && s0 > h) __hip_atomic_fetch_max(seg_hint, s0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return s0;
  };
  int known = -1;   // wave 0: the last segment seen with all its flags
  while (true) {
    // wave 0: the next piece to copy, s_copy = (segment or -1 none now / -2
    // done, first unit, end unit); s_copy[3..5] = the claim's units [p0, p1)
    // and the segment holding p0, kept across calls
    if (tid < 64) {
      int state = -1, c0 = 0, c1 = 0;
      int p0 = s_copy[3], p1 = s_copy[4], ps = s_copy[5];
      if (p0 >= p1) {
        bool take = true;
        if (!wait) {
          const int u = __hip_atomic_load(next_unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (u >= n_units) {
            take = false;
            state = -2;
          } else {
            const int sg = find_seg(u, ps);
            if (sg != known && !tiles_ready(sg)) {
              take = false;
            } else {
              known = sg;
              // a claim races with others and may land past u: take one only
              // with two claims' worth of ready units ahead (else the units
              // would wait here, claimed, while this workgroup runs a tile)
              if (u + 2 * kClaimUnits > unit_end(sg) && sg + 1 < n_seg && !tiles_ready(sg + 1)) take = false;
            }
            ps = sg;   // starts at or below u, so at or below every later claim
          }
        }
        if (take) {
          int t = 0;
          // the last units are spread over at least 64 workgroups: a claim is
          // at most an even share of the units left (a small copy, or the
          // last segments, which turn ready while most workgroups still run
          // their last tiles, would otherwise fall to a few workgroups). Also
          // between tiles, not only once the tiles have run out: on MI355X
          // this took the fine-grained layer's exposed copy from 9 to 4 us
          // (of a 71 us bulk copy) for 1% of the role-switching launch.
          const int left = n_units - __hip_atomic_load(next_unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int nc = max(1, min(kClaimUnits, left / 64));
          if (lane == 0) t = __hip_atomic_fetch_add(next_unit, nc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          t = __shfl(t, 0);
          if (t >= n_units) {
            state = -2;
          } else {
            p0 = t;
            p1 = min(t + nc, n_units);
            ps = find_seg(p0, ps);
          }
        }
      }
      if (p0 < p1) {
        const int sg = ps;
        bool ready = sg == known;
        if (!ready) {
          const uint64_t t_start = wall_clock64();
          while (true) {
            ready = tiles_ready(sg);
            if (ready || !wait) break;
            if (wall_clock64() - t_start > a.wait_ticks) {
              if (lane == 0) {
                int expected = 0;
                __hip_atomic_compare_exchange_strong(const_cast<int32_t*>(a.meta) + META_STATUS, &expected,
                                                     MOE_ERR_TIMEOUT, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
              }
              state = -2;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        if (ready) {
          known = sg;
          state = sg;
          c0 = p0;
          c1 = min(p1, unit_end(sg));
          p0 = c1;
          if (p0 < p1) ps = sg + 1;   // the claim goes on in the next segment
        }
      }
      if (lane == 0) {
        s_copy[0] = state; s_copy[1] = c0; s_copy[2] = c1;
        s_copy[3] = p0; s_copy[4] = p1; s_copy[5] = ps;
      }
    }
    __syncthreads();
    const int sg = s_copy[0], c0 = s_copy[1], c1 = s_copy[2];
    __syncthreads();
    if (sg < 0) return;
    if (!MOE_DEVICE_SCOPE_PUBLISH) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // units relative to the segment, as 16-byte words of its rows
    constexpr uint32_t kUnitWords = kCopyUnitBytes / 16;
    const int base = a.seg_unit0[sg];
    const uint32_t seg_words = (uint32_t)a.seg_rows[sg] * (uint32_t)(a.Nout / 8);
    copy_words<NT>(a, sg, (uint32_t)(c0 - base) * kUnitWords, min((uint32_t)(c1 - base) * kUnitWords, seg_words),
                   tid);
    // these copies have completed: the latest such stamp is the transfer's end
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) stamp_max(a.meta, META_T_CONS);
  }
}

template <int BM, int BN, int BK, int NS, int WM, int WN, int EPI, bool COPY = false, int GATHER = 0,
          bool CONS = false>
__global__ __launch_bounds__(WM * WN * 64, 1) void k_gemm(const GemmArgs a) {
  using C = Tile<BM, BN, BK, NS, WM, WN>;
  static_assert(!CONS || C::LDS_ELEMS * 2 >= kSegLdsBytes, "consumer tables fit the tile's LDS");
  static_assert(EPI != EPI_GATED || C::FN % 2 == 0, "gated tiles pair W1/W3 32-column blocks per wave");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];
  __shared__ int s_item[5];   // tile, chunk, nsplit, slot, queue
  __shared__ int s_copy[6];   // copy duty: the piece to copy, this workgroup's claim
  // output projection: the chunks of a split tail tile share its reduction
  constexpr bool kShared = EPI == EPI_PLAIN;
  constexpr int kBlocks = C::FM * C::FN;   // 32x32 accumulator blocks per wave
  constexpr int kMaxSplit = kShared ? (kMaxSplitShared < kBlocks ? kMaxSplitShared : kBlocks) : kMaxSplitSerial;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int K = a.K;
  const int nk = K / BK;

  // the other launch's queue and tail counters (this launch's were cleared by it)
  if (blockIdx.x == 0 && tid < kXcds * kCtrStride) a.other_ctr[tid] = 0;
  if (blockIdx.x == 0 && tid < kCtrStride) a.other_copy[tid] = 0;
  if constexpr (EPI != EPI_PLAIN) {
    // the output projection's clock stamps, and its ready flags: every call
    // starts from zero flags, so a replayed call (same epoch) never sees a
    // previous call's flags
    if (blockIdx.x == 0 && tid < 4) const_cast<int32_t*>(a.meta)[META_T_PROD + tid] = 0;
    if (a.flags != nullptr) {
      const int nf = a.meta[META_NTILES] * a.flags_n;
      for (int i = blockIdx.x * C::NT + tid; i < nf; i += gridDim.x * C::NT) a.flags[i] = 0u;
    }
  }
  const int px = max(1, a.px > 0 ? a.px : ((int)gridDim.x - a.meta[META_CAUTO]) / kXcds);
  if (a.trace != nullptr && blockIdx.x == 0 && tid == 0) a.trace[0] = wall_clock64();
  if (COPY && tid == 0) { s_copy[3] = 0; s_copy[4] = 0; s_copy[5] = 0; }   // no claim yet
  if constexpr (CONS) {
    const int n_cons = a.n_cons > 0 ? a.n_cons : a.meta[META_CAUTO];
    if ((int)blockIdx.x < n_cons) {
      // a copy of fewer units than four per consumer workgroup goes one unit
      // per workgroup, so as many workgroups as it has units share it
      if (a.meta[META_NUNITS] < 4 * n_cons)
        consume<C::NT, 1, (int)(kCopyUnitBytes / 16 / C::NT)>(a.cons, blockIdx.x, n_cons,
                                                               reinterpret_cast<int*>(lds), s_copy);
      else
        consume<C::NT, 4, 32>(a.cons, blockIdx.x, n_cons, reinterpret_cast<int*>(lds), s_copy);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this workgroup's copies have completed
      __syncthreads();
      if (tid == 0) stamp_max(a.meta, META_T_CONS);
      // its segments copied, the workgroup joins the producer for the tiles
      // still queued (the local ones come last); the tail split stays sized
      // for the producer's n_cu - c workgroups, so the bits do not change
    }
  }

  // DMA lane geometry: lane -> (row inside the instruction, physical chunk).
  // The swizzle depends on the tile row modulo 2*RPI, so one byte offset per
  // parity of the instruction's row block covers every DMA of A and of B.
  const int d_row = lane / C::CPR;
  const int d_pch = lane % C::CPR;
  uint32_t lane_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    lane_off[par] = (uint32_t)(d_row * K * 2 + swz<C::CPR>(par * C::RPI + d_row, d_pch) * 16);
  // MFMA fragment geometry (v_mfma_f32_16x16x32_bf16): lane l reads row
  // (l & 15) + 16 i of A (column 16 j of B) and the 8 k's of logical chunk
  // 4 s + (l >> 4) of k32 substep s. The swizzle only depends on the row mod
  // 16 and XORs the chunk index, so one lane offset f_off (substep 0) covers
  // every 16-row block of A and B; substep s reads f_off ^ 32 s (chunk ^ 4).
  // The instances without copy duty keep the four sums (per substep and
  // operand) in registers; the copying one, whose copy state leaves it no
  // room for them, forms them per substep from f_off (kept in registers,
  // they had spilled into its k-loop, and the reload's vmcnt wait drained
  // the DMA ring every stage: its output projection 25-30% slower).
  static_assert(C::CPR == 8 && C::WTM % 16 == 0 && C::WTN % 16 == 0, "fragment offsets assume BK = 64");
  const int f_off = (lane & 15) * BK + swz<C::CPR>(lane & 15, lane >> 4) * 8;
  const int a_woff = __builtin_amdgcn_readfirstlane(wm * C::WTM * BK);
  const int b_woff = __builtin_amdgcn_readfirstlane(BM * BK + wn * C::WTN * BK);
  int a_off[2], b_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    a_off[s] = a_woff + (f_off ^ (s * 32));
    b_off[s] = b_woff + (f_off ^ (s * 32));
  }

  const int n_rt = a.meta[META_NTILES];   // row tiles, in schedule positions
  const int n_rrt = a.meta[META_NRTILES];  // the first n_rrt of them hold a remote band
  const int m_pad = GATHER ? a.meta[META_MPAD] : 0;
  moe_i32x4 a_rsrc = {0, 0, 0, 0};
  if constexpr (GATHER == 2) {
    // x as a raw buffer: a_nrows rows of K bf16 (the host checks the size fits below kBufOutOfRange)
    const uint64_t xa = reinterpret_cast<uint64_t>(a.A);
    a_rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)xa);
    a_rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(xa >> 32));
    a_rsrc[2] = __builtin_amdgcn_readfirstlane((int)((uint32_t)a.a_nrows * (uint32_t)(K * 2)));
    a_rsrc[3] = 0x00020000;   // 32-bit data format, no swizzle, no stride: byte-addressed raw buffer
  }
  int q = xcc_id(), tried = 0;
  while (true) {
    if constexpr (COPY) copy_duty<C::NT>(a, false, tid, s_copy);
    if (tid == 0) {
      Item it{-1, 0, 1, 0};
      while (tried < kXcds) {
        const int i = __hip_atomic_fetch_add(a.my_ctr + q * kCtrStride, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        it = queue_item(a, n_rt, n_rrt, q, i, px, nk, kMaxSplit, kShared ? kMinSplitStepsSparse : kMinSplitSteps);
        if (it.tile >= 0) break;
        q = (q + 1) & (kXcds - 1);
        ++tried;
      }
      s_item[0] = it.tile; s_item[1] = it.chunk; s_item[2] = it.nsplit; s_item[3] = it.slot;
      s_item[4] = q;
    }
    __syncthreads();
    const int tile = s_item[0];
    if (tile < 0) {
      if constexpr (COPY) copy_duty<C::NT>(a, true, tid, s_copy);
      break;
    }
    const int chunk = __builtin_amdgcn_readfirstlane(s_item[1]);
    const int nsplit = __builtin_amdgcn_readfirstlane(s_item[2]);
    const int slot = __builtin_amdgcn_readfirstlane(s_item[3]);
    const int iq = __builtin_amdgcn_readfirstlane(s_item[4]);
    __syncthreads();   // everyone has read s_item before thread 0 may overwrite it
    // this item's k-steps
    const int kb = chunk * nk / nsplit;
    const int nkc = (chunk + 1) * nk / nsplit - kb;

    const int tile_u = __builtin_amdgcn_readfirstlane(tile);
    const int st = tile_u / a.tiles_n;           // schedule position of the row tile
    const int tn = tile_u - st * a.tiles_n;
    const int rt = a.tile_sched[st];             // row tile (layout order)
    const int row0 = a.tile_row0[rt];
    const int e = a.tile_expert[rt];
    const int vrows = a.tile_rows[rt];           // rows to store (the rest is the next expert's)
    const int fidx = rt * a.tiles_n + tn;        // flag / trace index

    // wave-uniform global bases of this wave's DMA instructions (k offset added per stage);
    // gathered A: each lane's own source row instead, its swizzled chunk included.
    // A rows past the last 32-row block holding stored rows feed no MFMA: their
    // DMA instructions still run (the stage waits count them) but read the
    // tile's first rows (or the zero row) again, which the L2 already holds.
    const int act_rows = min(BM, (vrows + 31) & ~31);
    const char* abase[C::A_PW];
    const char* bbase[C::B_PW];
    // GATHER 2: 32-bit offsets into x's buffer resource, padding rows at an
    // offset past its end (zeros, no memory read)
    uint32_t aoff[GATHER == 2 ? C::A_PW : 1];
    if constexpr (GATHER) {
      // every source index is loaded before any is used (one wait), with
      // unconditional clamped loads
      int src[C::A_PW];
#pragma unroll
      for (int i = 0; i < C::A_PW; ++i)
        src[i] = a.a_rows[min(row0 + (wave_u * C::A_PW + i) * C::RPI + d_row, m_pad - 1)];
#pragma unroll
      for (int i = 0; i < C::A_PW; ++i) {
        const int blk = wave_u * C::A_PW + i;
        const int r = row0 + blk * C::RPI + d_row;
        const bool real = r < m_pad && (unsigned)src[i] < (unsigned)a.a_nrows && blk * C::RPI < act_rows;
        const uint32_t chunk_off = (uint32_t)swz<C::CPR>((blk & 1) * C::RPI + d_row, d_pch) * 16;
        if constexpr (GATHER == 2) {
          aoff[i] = real ? (uint32_t)src[i] * (uint32_t)(K * 2) + chunk_off : kBufOutOfRange;
        } else {
          const uint64_t rp = real ? reinterpret_cast<uint64_t>(a.A) + (uint64_t)(uint32_t)src[i] * (uint64_t)(K * 2)
                                   : reinterpret_cast<uint64_t>(a.a_zero);
          abase[i] = reinterpret_cast<const char*>(rp + chunk_off);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_PW; ++i) {
        const int rb = (wave_u * C::A_PW + i) * C::RPI;
        abase[i] = reinterpret_cast<const char*>(a.A) + ((size_t)(row0 + (rb < act_rows ? rb : 0)) * K) * 2;
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PW; ++i) {
      const int r = (wave_u * C::B_PW + i) * C::RPI;   // first B-tile row of the instruction
      int wrow;
      const uint16_t* w;
      if constexpr (EPI == EPI_GATED) {
        w = ((r >> 5) & 1) ? a.B1 : a.B0;                // 32-row blocks alternate W1 / W3
        wrow = tn * (BN / 2) + (r >> 6) * 32 + (r & 31);
      } else {
        w = a.B0;
        wrow = tn * BN + r;
      }
      bbase[i] = reinterpret_cast<const char*>(w) + ((size_t)e * a.Nw * K + (size_t)wrow * K) * 2;
    }
    const uint32_t lds0 = lds_addr(lds);
    // this wave's DMA instructions q in [q0, q1) of stage kt: q < A_PW are its
    // A rows, the rest its B rows
    auto issue_part = [&](int kt, int q0, int q1) {
      const uint32_t st = lds0 + (uint32_t)((kt % NS) * C::STAGE * 2);
      const size_t ko = (size_t)(kb + kt) * BK * 2;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        if (q < q0 || q >= q1) continue;
        if (q < C::A_PW) {
          const int blk = wave_u * C::A_PW + q;
          if constexpr (GATHER == 2) dma16_buf(aoff[q] + (uint32_t)ko, a_rsrc, st + (uint32_t)(blk * C::RPI * BK * 2));
          else if constexpr (GATHER) dma16_v(abase[q] + ko, st + (uint32_t)(blk * C::RPI * BK * 2));
          else dma16(abase[q] + ko, lane_off[blk & 1], st + (uint32_t)(blk * C::RPI * BK * 2));
        } else {
          const int blk = wave_u * C::B_PW + (q - C::A_PW);
          dma16(bbase[q - C::A_PW] + ko, lane_off[blk & 1], st + (uint32_t)((BM + blk * C::RPI) * BK * 2));
        }
      }
    };
    auto issue = [&](int kt) { issue_part(kt, 0, C::LPW); };

    // accumulators per 32x32 block (i, j) of the wave tile, as four 16x16
    // MFMA results: acc[i][j][sub][rr] is row 32 i + 16 (sub >> 1) + 4 (l >> 4)
    // + rr, column 32 j + 16 (sub & 1) + (l & 15); r = 4 sub + rr runs over a
    // block's 16 values
    f32x4 acc[C::FM][C::FN][4];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r >> 2][r & 3] = 0.f;

    // k-loop, software-pipelined:
    //  * all NS ring slots are in flight: stage kt+NS is issued into stage kt's
    //    slot as soon as every wave has finished reading stage kt, half of a
    //    wave's DMA instructions after the barrier and half after the step's
    //    last MFMAs (one burst of all of them made the issuing waves queue
    //    behind the texture path: the first projection took 4% longer at
    //    K = 4096; a third or more of them in the next step, less time to land);
    //  * a stage is four quarters: k32 substep s = q / 2 against half h = q % 2
    //    of the wave's 16-column B blocks (v_mfma_f32_16x16x32_bf16; 16 x 16
    //    MFMAs interleave with the DMA and fragment reads better than 32 x 32
    //    ones of the same flops: both projections 3-5% faster on the
    //    Mixtral-shaped shares, the extra fragment registers spill only in
    //    the item set-up and the epilogue). Fragments are
    //    double-buffered: quarter q+1's load while quarter q's MFMAs run
    //    (quarter (s, 0) loads substep s's A blocks with its B half);
    //  * the stage barrier sits before the last quarter's MFMAs (whose
    //    fragments are already in registers), so stage kt+1's first
    //    fragments load while they run.
    constexpr int KK = BK / 16;   // quarters per stage
    bf16x8 fa[2][2 * C::FM], fb[2][C::FN];
    auto load_frags = [&](int kt, int q, int buf) {
      const uint16_t* st = lds + (kt % NS) * C::STAGE;
      const int s = q >> 1, h = q & 1;
      const int ao = COPY ? a_woff + (f_off ^ (s * 32)) : a_off[s];
      const int bo = COPY ? b_woff + (f_off ^ (s * 32)) : b_off[s];
      if (h == 0) {
#pragma unroll
        for (int i = 0; i < 2 * C::FM; ++i)
          fa[s & 1][i] = *reinterpret_cast<const bf16x8*>(st + ao + i * 16 * BK);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        fb[buf][j] = *reinterpret_cast<const bf16x8*>(st + bo + (h * C::FN + j) * 16 * BK);
    };
    // 16-row blocks of this wave that hold stored rows (a short last row tile
    // of an expert skips the MFMAs of the blocks past them; with 16-row bands
    // the last block may be the next expert's rows, computed, not stored)
    const int fm_act = __builtin_amdgcn_readfirstlane(min(2 * C::FM, max(0, (vrows - wm * C::WTM + 15) / 16)));
    auto mfmas = [&](int q, int buf, auto partial) {
      const int s = q >> 1, h = q & 1;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int jb = h * C::FN + j;   // 16-column block of the wave tile
#pragma unroll
        for (int i = 0; i < 2 * C::FM; ++i) {
          if (decltype(partial)::value && i >= fm_act) continue;
          f32x4& d = acc[i >> 1][jb >> 1][(i & 1) * 2 + (jb & 1)];
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][i], fb[buf][j], d, 0, 0, 0);
        }
      }
    };

    // previous tile's stores must not be counted by the stage waits below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nkc) issue(s);
    if (nkc >= NS) wait_vm_barrier<(NS - 1) * C::LPW>();
    else wait_vm_barrier<0>();
    load_frags(0, 0, 0);
    auto kloop = [&](auto partial) {
      for (int kt = 0; kt < nkc; ++kt) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
          load_frags(kt, kk + 1, (kk + 1) & 1);
          mfmas(kk, kk & 1, partial);
        }
        const bool more = kt + NS < nkc;
        if (kt + 1 < nkc) {
          if (kt + NS <= nkc) wait_vm_barrier<(NS - 2) * C::LPW>();
          else wait_vm_barrier<0>();
          if (more) issue_part(kt + NS, 0, C::LPW / 2);
          load_frags(kt + 1, 0, 0);
        }
        mfmas(KK - 1, (KK - 1) & 1, partial);
        if (more) issue_part(kt + NS, C::LPW / 2, C::LPW);
      }
    };
    if (fm_act == 2 * C::FM) kloop(std::false_type{});
    else kloop(std::true_type{});

    if (a.dbg_seed != 0u) {
      // test knob: a seeded delay before this item's results go out
      uint32_t h = a.dbg_seed ^ ((uint32_t)fidx * 0x9E3779B1u) ^ ((uint32_t)chunk * 0x85EBCA77u);
      h ^= h >> 15; h *= 0x2C1B3C6Du; h ^= h >> 12;
      const int n = __builtin_amdgcn_readfirstlane((int)(h % 24u));
      for (int z = 0; z < n; ++z) __builtin_amdgcn_s_sleep(127);
    }

    // ---- epilogue
    // Rows of a tile holding a remote band are published for the copying
    // roles (sec. 3.3.1: store, then flag): device-scope 16-byte stores,
    // which write through this XCD's L2, and once they have completed the
    // tile's ready flag. Tiles holding only this rank's own rows are never
    // copied: plain stores and no flag.
    const bool pub = (EPI == EPI_PLAIN) && a.flags != nullptr && st < n_rrt;
    constexpr int OUTW = (EPI == EPI_GATED) ? BN / 2 : BN;
    constexpr int LROW = OUTW + 8;
    constexpr int CH = OUTW / 8;   // 16-byte chunks per output row
    const int ncol = lane & 15;          // column inside a 16 x 16 result
    const int mrow = (lane >> 4) * 4;    // first of the lane's four rows in it
    uint16_t* cbase = a.C + (size_t)row0 * a.Nout + (size_t)tn * OUTW;
    // accumulator blocks q in [q0, q1) of every wave (q = j * FM + i) -> LDS ->
    // the tile's rows (layout at acc above). The bf16 tile is staged in LDS
    // (row stride OUTW + 8 keeps the four row groups of a store on disjoint
    // banks) and leaves as 16-byte row chunks.
    auto store_blocks = [&](int q0, int q1) {
      __syncthreads();   // every wave is done reading the ring (or the last staging)
      if constexpr (EPI == EPI_GATED) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int p = 0; p < C::FN / 2; ++p) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int sub = r >> 2, rr = r & 3;
              const int c = wn * (C::WTN / 2) + p * 32 + (sub & 1) * 16 + ncol;
              const int m = wm * C::WTM + i * 32 + (sub >> 1) * 16 + mrow + rr;
              lds[m * LROW + c] = f32_to_bf16_rne(silu_f32(acc[i][2 * p][sub][rr]) * acc[i][2 * p + 1][sub][rr]);
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if (j * C::FM + i < q0 || j * C::FM + i >= q1) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int sub = r >> 2, rr = r & 3;
              const int c = wn * C::WTN + j * 32 + (sub & 1) * 16 + ncol;
              const int m = wm * C::WTM + i * 32 + (sub >> 1) * 16 + mrow + rr;
              float v = acc[i][j][sub][rr];
              if constexpr (EPI == EPI_SILU) v = silu_f32(v);
              lds[m * LROW + c] = f32_to_bf16_rne(v);
            }
          }
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(cbase, (uint32_t)vrows * (uint32_t)a.Nout * 2u);
      auto store_chunk = [&](int m, int cc) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + m * LROW + cc * 8);
#if MOE_DEVICE_SCOPE_PUBLISH
        if (pub) {
          store16_device(rs, ((uint32_t)m * (uint32_t)a.Nout + (uint32_t)(cc * 8)) * 2u, v);
          return;
        }
#endif
        *reinterpret_cast<u32x4*>(cbase + (size_t)m * a.Nout + cc * 8) = v;
      };
      const int nq = q1 - q0;
      if (nq == kBlocks) {
#pragma unroll 4
        for (int x = tid; x < vrows * CH; x += C::NT) store_chunk(x / CH, x - (x / CH) * CH);
      } else {
        // a share of a split tile: blocks q0..q1-1 of every wave, 32 rows x 4 chunks each
        for (int x = tid; x < C::NW * nq * 128; x += C::NT) {
          const int wb = x / (nq * 128);
          const int rem = x - wb * (nq * 128);
          const int q = q0 + (rem >> 7);
          const int m = (wb / WN) * C::WTM + (q % C::FM) * 32 + ((rem & 127) >> 2);
          if (m < vrows) store_chunk(m, ((wb % WN) * C::WTN + (q / C::FM) * 32) / 8 + (rem & 3));
        }
      }
    };
    // the tile's rows are all stored (by this workgroup or, for a split tile,
    // by the chunks before it): raise the flag, stamp the tile's end
    auto finish_tile = [&]() {
      if (pub) {
#if MOE_DEVICE_SCOPE_PUBLISH
        // all of this workgroup's device-scope stores have completed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(a.flags + fidx, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0)
          __hip_atomic_store(a.flags + fidx, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
#endif
      } else if (COPY || CONS || (EPI == EPI_PLAIN && a.trace != nullptr)) {
        __syncthreads();
      }
      if constexpr (COPY || CONS) {
        if (tid == 0) stamp_max(a.meta, META_T_PROD);
      }
      if (EPI == EPI_PLAIN && a.trace != nullptr && tid == 0) a.trace[8 + fidx] = wall_clock64();
    };
    // fp32 partials of split tail tiles: lane-native layout ((wave * FM + i) *
    // FN + j) * 8 + pair, then 64 lanes x 2 floats
    const uint64_t* part0 = reinterpret_cast<const uint64_t*>(a.partial) +
                            (size_t)(iq * kTailSlots + slot - chunk) * (BM * BN / 2) +
                            (size_t)wave * (C::FM * C::FN * 512) + lane;
    // acc of blocks [q0, q1) = the sum of every chunk's partials, in chunk order
    // (so the tile's bits do not depend on the order of arrivals or on who sums)
    auto reduce_blocks = [&](int q0, int q1) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r >> 2][r & 3] = 0.f;
      if (kShared && q1 - q0 < kBlocks) {
        // a few blocks: the partials of up to four chunks of a block in flight
        // at once (clamped loads, so none is predicated), added in chunk order
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const int q = j * C::FM + i;
            if (q < q0 || q >= q1) continue;
            for (int cb = 0; cb < nsplit; cb += 4) {
              uint64_t v[4][8];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const uint64_t* part = part0 + (size_t)min(cb + u, nsplit - 1) * (BM * BN / 2);
#pragma unroll
                for (int r = 0; r < 8; ++r)
                  v[u][r] = __hip_atomic_load(part + ((i * C::FN + j) * 8 + r) * 64, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
              }
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (cb + u >= nsplit) break;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                  acc[i][j][r >> 1][(r & 1) * 2] += __uint_as_float((uint32_t)v[u][r]);
                  acc[i][j][r >> 1][(r & 1) * 2 + 1] += __uint_as_float((uint32_t)(v[u][r] >> 32));
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
      } else {
        for (int c2 = 0; c2 < nsplit; ++c2) {
          const uint64_t* part = part0 + (size_t)c2 * (BM * BN / 2);
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const uint64_t v = __hip_atomic_load(part + ((i * C::FN + j) * 8 + r) * 64, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                acc[i][j][r >> 1][(r & 1) * 2] += __uint_as_float((uint32_t)v);
                acc[i][j][r >> 1][(r & 1) * 2 + 1] += __uint_as_float((uint32_t)(v >> 32));
              }
              // one 32x32 block of loads in flight at a time (the accumulators stay live)
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
    };

    // Split tail tile: publish this chunk's accumulators as a partial tile
    // (device-scope stores), wait for them to complete, count the arrival.
    //  * first projection: the last chunk to arrive sums all partials and
    //    finishes the tile; the others are done;
    //  * output projection: the accumulator blocks are cut into nsplit
    //    shares. A chunk that sees every chunk arrive (waiting at most
    //    tail_wait_ticks) claims its own share; the last chunk to arrive
    //    claims its own and then every share still unclaimed, so no chunk
    //    depends on another workgroup being resident. Each share is summed
    //    in chunk order and stored by the one chunk that claimed it; the
    //    chunk storing the tile's last share raises the flag.
    const bool split = nsplit > 1;
    constexpr bool kSplitShares = kShared;
    bool last_arrival = true;
    int32_t* tail_ctr = a.my_ctr + iq * kCtrStride + 1 + slot / nsplit;
    if (split) {
      uint64_t* mine = reinterpret_cast<uint64_t*>(a.partial) +
                       (size_t)(iq * kTailSlots + slot) * (BM * BN / 2) +
                       (size_t)wave * (C::FM * C::FN * 512) + lane;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const uint64_t v = (uint64_t)__float_as_uint(acc[i][j][r >> 1][(r & 1) * 2]) |
                               ((uint64_t)__float_as_uint(acc[i][j][r >> 1][(r & 1) * 2 + 1]) << 32);
            __hip_atomic_store(mine + ((i * C::FN + j) * 8 + r) * 64, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#if !MOE_DEVICE_SCOPE_PUBLISH
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#endif
      __syncthreads();
      if (tid == 0)
        s_item[0] = __hip_atomic_fetch_add(tail_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int arrived = s_item[0];
      __syncthreads();   // s_item is rewritten below and by the next item
      last_arrival = arrived == nsplit - 1;
      if (!kSplitShares && !last_arrival) continue;
      if (kSplitShares && !last_arrival) {
        if (tid == 0) {
          int ok = 1;
          const uint64_t t_start = wall_clock64();
          while (__hip_atomic_load(tail_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nsplit) {
            if (wall_clock64() - t_start > a.tail_wait_ticks) { ok = 0; break; }
            __builtin_amdgcn_s_sleep(2);
          }
          s_item[0] = ok;
        }
        __syncthreads();
        const int ok = s_item[0];
        __syncthreads();
        if (!ok) continue;   // the last chunk to arrive takes this share
      }
#if !MOE_DEVICE_SCOPE_PUBLISH
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
    }
    // the tile's shares this workgroup stores: a whole tile (or the first
    // projection's reduced split tile) is one share of every block
    const int n_sh = (kSplitShares && split) ? nsplit : 1;
    for (int k2 = 0; k2 < n_sh; ++k2) {
      if (k2 > 0 && !last_arrival) break;
      int q0 = 0, q1 = kBlocks;
      if (kSplitShares && split) {
        const int sh = chunk + k2 < nsplit ? chunk + k2 : chunk + k2 - nsplit;
        uint32_t* claimed = reinterpret_cast<uint32_t*>(a.my_ctr + iq * kCtrStride + 1 + kTailTiles + slot / nsplit);
        if (tid == 0)
          s_item[0] = (int)((__hip_atomic_fetch_or(claimed, 1u << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >>
                             sh) & 1u);
        __syncthreads();
        const int taken = s_item[0];
        __syncthreads();
        if (taken) continue;
        q0 = sh * kBlocks / nsplit;
        q1 = (sh + 1) * kBlocks / nsplit;
      }
      if (split) reduce_blocks(q0, q1);
      store_blocks(q0, q1);
      bool done = true;
      if (kSplitShares && split) {
        // count the stored share; the tile is done with its last share
#if MOE_DEVICE_SCOPE_PUBLISH
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#else
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#endif
        __syncthreads();
        if (tid == 0)
          s_item[0] = __hip_atomic_fetch_add(tail_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        done = s_item[0] == 2 * nsplit - 1;
        __syncthreads();
#if !MOE_DEVICE_SCOPE_PUBLISH
        if (done) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
      }
      if (done) finish_tile();
    }
  }
}

template <int BM, int BN, int BK, int NS, int WM, int WN, int EPI>
static hipError_t launch_t(const GemmArgs& a, int grid, hipStream_t st) {
  if constexpr (EPI == EPI_PLAIN) {
    if (a.copy_duty) {
      hipLaunchKernelGGL((k_gemm<BM, BN, BK, NS, WM, WN, EPI, true>), dim3(grid), dim3(WM * WN * 64), 0, st, a);
      return hipGetLastError();
    }
    if (a.n_cons != 0) {
      hipLaunchKernelGGL((k_gemm<BM, BN, BK, NS, WM, WN, EPI, false, false, true>), dim3(grid),
                         dim3(WM * WN * 64), 0, st, a);
      return hipGetLastError();
    }
  } else {
    if (a.a_rows != nullptr && (uint64_t)a.a_nrows * (uint64_t)a.K * 2 < (uint64_t)kBufOutOfRange) {
      hipLaunchKernelGGL((k_gemm<BM, BN, BK, NS, WM, WN, EPI, false, 2>), dim3(grid), dim3(WM * WN * 64), 0,
                         st, a);
      return hipGetLastError();
    }
    if (a.a_rows != nullptr) {
      hipLaunchKernelGGL((k_gemm<BM, BN, BK, NS, WM, WN, EPI, false, 1>), dim3(grid), dim3(WM * WN * 64), 0,
                         st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemm<BM, BN, BK, NS, WM, WN, EPI>), dim3(grid), dim3(WM * WN * 64), 0, st, a);
  return hipGetLastError();
}

// XCD grid and block shape for a launch with tiles_n column tiles: at most
// 4 column groups (so each XCD takes every other row tile); blocks of 32
// tiles (one round of an XCD's 32 workgroups), or of 64 in the first
// projection (16 row tiles x 4 column tiles). Measured against 8 column
// groups and 32-tile blocks: the first projection 1-3% faster on the five
// workloads; 64-tile blocks in the output projection make its row tiles
// finish in coarser bursts, and the consumer fell behind (workload 4).
static inline void set_xcd_grid(GemmArgs& a, bool first_projection) {
  a.xn = a.tiles_n >= 8 ? 4 : (a.tiles_n >= 2 ? 2 : 1);
  a.xb = kXcds / a.xn;
  const int nn = (a.tiles_n + a.xn - 1) / a.xn;
  a.gq = nn < 4 ? nn : 4;
  a.gp = (first_projection ? 64 : 32) / a.gq;
}

// per-shape tile table (row tiles of kTileM rows; BN from the geometry).
// 8 waves (two per SIMD) let one wave's MFMAs cover the other's LDS and DMA
// waits; measured on MI355X for the Mixtral-shaped projections.
template <int EPI>
static hipError_t dispatch(GemmArgs a, int bm, int bn, int grid, hipStream_t st) {
  set_xcd_grid(a, EPI != EPI_PLAIN);
  if (bm == 256 && bn == 256) return launch_t<256, 256, 64, 2, 4, 2, EPI>(a, grid, st);
  if (bm == 256 && bn == 128) return launch_t<256, 128, 64, 3, 4, 2, EPI>(a, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm1(const Geometry& g, const uint16_t* a_src, const int32_t* a_rows,
                        const uint16_t* a_zero, const uint16_t* w1, const uint16_t* w3, uint16_t* h,
                        const moe_plan_t& p, uint32_t* flags, int grid, const GemmKnobs& kn, hipStream_t st) {
  GemmArgs a{};
  a.dbg_seed = kn.delay_seed;
  a.dbg_reverse = kn.reverse;
  a.tail_wait_ticks = kn.tail_wait_ticks;
  a.A = a_src;
  a.a_rows = a_rows;
  a.a_zero = a_zero;
  a.a_nrows = g.R * g.T;
  a.B0 = w1;
  a.B1 = w3;
  a.C = h;
  a.meta = p.meta;
  a.tile_row0 = p.tile_row0;
  a.tile_expert = p.tile_expert;
  a.tile_rows = p.tile_rows;
  a.tile_sched = p.tile_sched;
  a.my_ctr = p.tile_ctr;
  a.other_ctr = p.tile_ctr + kXcds * kCtrStride;
  a.my_copy = p.tile_ctr + kCopyCtrOffset;
  a.other_copy = p.tile_ctr + kCopyCtrOffset + kCtrStride;
  a.partial = p.partial;
  a.flags = flags;
  a.flags_n = g.tiles2;
  a.trace = nullptr;
  a.epoch = 0;
  a.K = g.H;
  a.Nw = g.F;
  a.Nout = g.F;
  a.tiles_n = g.tiles1;
  a.px = grid / kXcds;
  return g.gated ? dispatch<EPI_GATED>(a, g.tile_m, g.bn1, grid, st)
                 : dispatch<EPI_SILU>(a, g.tile_m, g.bn1, grid, st);
}

hipError_t launch_gemm2(const Geometry& g, const uint16_t* h, const uint16_t* w2, uint16_t* y,
                        const moe_plan_t& p, uint32_t* flags, uint32_t epoch, uint64_t* trace,
                        int grid, int split_grid, const BufPtrs* copy_bufs, int n_cons,
                        const BufPtrs* cons_bufs, uint64_t wait_ticks, const GemmKnobs& kn, hipStream_t st) {
  GemmArgs a{};
  a.dbg_seed = kn.delay_seed;
  a.dbg_reverse = kn.reverse;
  a.tail_wait_ticks = kn.tail_wait_ticks;
  a.A = h;
  a.B0 = w2;
  a.B1 = nullptr;
  a.C = y;
  a.meta = p.meta;
  a.tile_row0 = p.tile_row0;
  a.tile_expert = p.tile_expert;
  a.tile_rows = p.tile_rows;
  a.tile_sched = p.tile_sched;
  a.my_ctr = p.tile_ctr + kXcds * kCtrStride;
  a.other_ctr = p.tile_ctr;
  a.my_copy = p.tile_ctr + kCopyCtrOffset + kCtrStride;
  a.other_copy = p.tile_ctr + kCopyCtrOffset;
  a.partial = p.partial;
  if (copy_bufs != nullptr) {
    a.copy_duty = 1;
    a.bufs = *copy_bufs;
    a.seg_tile0 = p.seg_tile0;
    a.seg_tile1 = p.seg_tile1;
    a.seg_unit0 = p.seg_unit0;
    a.seg_rows = p.seg_rows;
    a.seg_src_row = p.seg_src_row;
    a.seg_dst_row = p.seg_dst_row;
    a.seg_dest = p.seg_dest;
  }
  if (n_cons != 0) {
    a.n_cons = n_cons;
    a.cons = consumer_args(g, y, *cons_bufs, p, flags, epoch, trace, wait_ticks);
  }
  a.flags = flags;
  a.trace = trace;
  a.epoch = epoch;
  a.K = g.F;
  a.Nw = g.H;
  a.Nout = g.H;
  a.tiles_n = g.tiles2;
  a.px = split_grid > 0 ? split_grid / kXcds : 0;
  a.wait_ticks = wait_ticks;
  return dispatch<EPI_PLAIN>(a, g.tile_m, g.bn2, grid, st);
}

}  // namespace moe
