// Internal definitions shared by the gfx950 kernels and the host ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe_overlap.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// tokens per routing chunk: a chunk never spans two source ranks
constexpr int kChunk = 256;
// local experts per rank at most (the plan and the chunk histograms size LDS by it)
constexpr int kPlanMaxElRoute = 256;
// meta words in the workspace
// META_CAUTO: consumer CUs the plan kernel's evaluation of the CU-split model
// chose (MOE_CONSUMER_AUTO); META_PRED: its predicted time (double, two words).
// META_T_PROD / META_T_CONS: uint64 device clock stamps (two words each) of the
// overlapped output projection's last producer exit and last consumer completion
// META_HISTCTR: arrivals of the routing histogram blocks (zeroed by k_route)
enum { META_MPAD = 0, META_NBANDS = 1, META_NREMOTE = 2, META_NSEG = 3, META_STATUS = 4, META_NUNITS = 5,
       META_NTILES = 6, META_NRTILES = 7, META_CAUTO = 8, META_T_PROD = 16, META_T_CONS = 18,
       META_PRED = 20, META_HISTCTR = 22, META_WORDS = 64 };
// GEMM row-tile height: the producer computes tiles of this many rows over each
// expert's tb_m-aligned rows, independently of the (possibly smaller) band
constexpr int kTileM = 256;
// segments are also cut into copy units of this many bytes (the baseline bulk copy)
constexpr int kCopyUnitBytes = 65536;
// per-XCD tile queues of the two GEMM launches: counter (phase, xcd) at
// tile_ctr[(phase*8 + xcd) * 32]; then one block of kCtrStride words per
// phase for the role-switching copy (word 0: next segment to claim)
constexpr int kXcds = 8;
constexpr int kCtrStride = 32;
constexpr int kCtrWords = 2 * kXcds * kCtrStride + 2 * kCtrStride;
constexpr int kCopyCtrOffset = 2 * kXcds * kCtrStride;
// K-split tail tiles of a GEMM launch: per XCD queue at most kTailSlots chunks,
// each with a tb_m x 256 fp32 partial tile; word 1 + t of the XCD's counter
// block counts the arrivals of tail tile t
constexpr int kTailSlots = kCtrStride - 1;
// bound on every wait for a ready flag, in ticks of the 100 MHz constant
// clock, unless the context sets another (moe_ctx_set_wait_limit)
constexpr uint64_t kDefaultWaitTicks = 200000000ull;   // 2 s
// bound on a split tail chunk's wait for the other chunks of its tile in the
// output projection (100 MHz ticks); past it the chunk leaves its share to
// the last chunk to arrive
constexpr uint64_t kDefaultTailWaitTicks = 100000ull;   // 1 ms

struct Geometry {
  int32_t R, T, H, F, E, k, r_self, gated, gate_kind, tb_m, mgb;
  int32_t El;                 // local experts
  int32_t chunks_per_rank;    // ceil(T / kChunk)
  int32_t n_chunks;           // R * chunks_per_rank
  int64_t m_pad_max;
  int32_t max_bands;
  int64_t rows;               // packed-row bound of the band layout
  int32_t tile_m;             // GEMM row-tile height
  int32_t max_tiles;          // GEMM row tiles at most
  int32_t bn1;                // first projection: MFMA tile width (u and v columns for gated)
  int32_t bn1_out;            // first projection: h columns per tile
  int32_t bn2;                // output projection tile width
  int32_t tiles1;             // h column tiles per band
  int32_t tiles2;             // y column tiles per band
  int32_t max_flags;
  int32_t recv_rows_max;
};

// Byte offsets of the workspace sections (all 256-byte aligned).
struct WsLayout {
  size_t meta, chunk_counts, chunk_base, group_row, expert_base, recv_off;
  size_t band_row0, band_expert, band_dest, band_recv0, band_valid;
  size_t seg_band0, seg_nbands, seg_dest, seg_src_row, seg_dst_row, seg_rows;
  size_t row_src, recv_row, tile_ctr, slot_valid, seg_unit0, partial;
  size_t tile_row0, tile_expert, tile_rows, tile_sched, seg_tile0, seg_tile1;
  size_t zero_row;   // [H] bf16 zeros (written by the plan): padding rows of the gathered GEMM
  size_t total;
};

int make_geometry(const moe_shape_t* s, Geometry* g);
WsLayout ws_layout(const Geometry& g);
void plan_from_ws(const Geometry& g, void* ws, moe_plan_t* p);
uint16_t* zero_row_of(const Geometry& g, void* ws);

// combine-buffer pointers travel to kernels by value
struct BufPtrs { uint16_t* p[MOE_MAX_RANKS]; };

#define GLOBAL_AS __attribute__((address_space(1)))

// A raw buffer resource over `bytes` bytes at p (p wave-uniform; the words are
// taken from the first lane so they sit in scalar registers). 16-byte loads and
// stores through it take a per-lane 32-bit byte offset; loads at or past
// `bytes` return zeros and stores there are dropped, without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, 0x00020000);
}

// cache policy of a buffer access: sc1 = device scope. A device-scope store
// writes through this XCD's L2 to the device's coherence point; a
// device-scope load misses in this XCD's L2 unless the line is coherent, so
// it sees rows another XCD published that way.
constexpr int kCpolDevice = 16;

// 16-byte load of rows another workgroup published with device-scope stores
__device__ __forceinline__ u32x4 load16_device(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCpolDevice);
}

// 16-byte device-scope store (publication of a tile's rows)
__device__ __forceinline__ void store16_device(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCpolDevice);
}

__device__ __forceinline__ void store16_nt(u32x4* a, u32x4 v) {
  __builtin_nontemporal_store(v, (GLOBAL_AS u32x4*)a);
}

// ---- kernel launchers (enqueue only) ----
hipError_t launch_route(const Geometry& g, const float* logits, int32_t* ids, float* gates,
                        const moe_plan_t& p, hipStream_t st);
hipError_t launch_count(const Geometry& g, const int32_t* ids, int32_t* counts, const moe_plan_t& p,
                        hipStream_t st);
// the plan, the index of the routed rows (row_src with -1 for every padding
// row, recv_row) and the CU-split model for `calib` (META_CAUTO, META_PRED)
hipError_t launch_plan(const Geometry& g, const int32_t* counts, const int32_t* ids, const moe_plan_t& p,
                       uint16_t* zero_row, const moe_calib_t& calib, hipStream_t st);
// the rows into x_perm (nothing when x_perm is null)
hipError_t launch_gather(const Geometry& g, const uint16_t* x, uint16_t* x_perm, const moe_plan_t& p,
                         hipStream_t st);
// a_rows null: A = x_perm (packed rows); else A = x and packed row r reads x row
// a_rows[r] (a_zero for padding), the gather fused into the tile loads.
// flags (may be null): the output projection's ready flags, cleared here
// Test knobs of the GEMM launches (timing only, never the results):
// delay_seed != 0 delays each work item by a seeded number of sleeps before
// its stores; reverse walks the tile queues in reverse schedule order;
// tail_wait_ticks bounds how long a split tail chunk of the output projection
// waits for its tile's other chunks (past it the last chunk to arrive
// reduces its share).
struct GemmKnobs {
  uint32_t delay_seed;
  int reverse;
  uint64_t tail_wait_ticks;
};
hipError_t launch_gemm1(const Geometry& g, const uint16_t* a_src, const int32_t* a_rows,
                        const uint16_t* a_zero, const uint16_t* w1, const uint16_t* w3, uint16_t* h,
                        const moe_plan_t& p, uint32_t* flags, int grid, const GemmKnobs& kn, hipStream_t st);
// split_grid: the producer grid the K-split tail is sized for (the overlapped
// run's n_cu - c in both modes, so that both compute identical bits)
// copy_bufs: non-null gives the launch the consumer's duty as well (role
// switching): between tiles a workgroup copies every remote segment whose row
// tiles are all flagged, and once the tiles run out it drains the rest
// n_cons != 0: workgroups [0, n_cons) of the launch are the consumer (copying
// into cons_bufs), the others the producer (the CU-partition overlap in one
// launch); n_cons = -1 and split_grid = 0 take the plan's consumer count.
// wait_ticks bounds each wait of either copying role for a ready flag.
hipError_t launch_gemm2(const Geometry& g, const uint16_t* h, const uint16_t* w2, uint16_t* y,
                        const moe_plan_t& p, uint32_t* flags, uint32_t epoch, uint64_t* trace,
                        int grid, int split_grid, const BufPtrs* copy_bufs, int n_cons,
                        const BufPtrs* cons_bufs, uint64_t wait_ticks, const GemmKnobs& kn, hipStream_t st);
hipError_t launch_bulk_copy(const Geometry& g, const uint16_t* y, BufPtrs bufs,
                            const moe_plan_t& p, int grid, hipStream_t st);
hipError_t launch_combine(const Geometry& g, BufPtrs bufs, const uint16_t* y, const float* gates,
                          const moe_plan_t& p, uint16_t* out, hipStream_t st);

// ---- device helpers ----
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

}  // namespace moe
