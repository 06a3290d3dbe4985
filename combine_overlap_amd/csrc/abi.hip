// Host side of the C ABI: argument validation (always before any HIP call),
// workspace layout, and the launch order of the share's kernels.
#include <string.h>

#include "common.hpp"
#include "partition_model.hpp"

#include <mutex>

#ifndef MOE_BULK_WG_PER_CU
#define MOE_BULK_WG_PER_CU 4   // workgroups per CU of the baseline's bulk copy
#endif

// ---- scratch of moe_expert_forward_noalloc ------------------------------
// The K-split partial tiles and the tile-queue / tail / copy counters of the
// two GEMM launches, in a file-scope device array instead of the caller's
// workspace, for callers that cannot allocate. Each GPU holds its own copy
// until the process ends. Host code never uses the array's name as an
// address: the per-device address comes from hipGetSymbolAddress (taken
// once per device in moe_ctx_create, with that device current).
constexpr size_t kScratchCtrBytes = 4096;   // counters (moe::kCtrWords int32)
constexpr size_t kScratchPartialBytes = (size_t)moe::kXcds * moe::kTailSlots * moe::kTileM * 256 * 4;
constexpr size_t kScratchBytes = kScratchCtrBytes + kScratchPartialBytes;   // 62 MiB + 4 KiB
static_assert(moe::kCtrWords * 4 <= (int)kScratchCtrBytes, "counters fit the scratch header");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// the current device's address of `scratch` (looked up once per device)
static int scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return MOE_OK;
}

// zeroes the scratch counters before a call (a kernel, not a memset node, so
// a captured call replays it)
__global__ void k_clear_scratch_ctr(int32_t* ctr, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) ctr[i] = 0;
}

struct moe_ctx {
  int device;
  int n_cu;
  int timing;               // 1: record tev[] in the forward
  int timed;                // a timed call has been enqueued
  int timed_mode;
  hipEvent_t tev[5];        // start, first projection end, producer end, consumer end, join
  uint64_t* trace;          // device timeline (see moe_ctx_set_trace) or null
  int32_t trace_flags;      // max_flags of the shape the trace was sized for
  const int32_t* timed_meta;   // workspace meta words of the last timed call (device stamps)
  uint64_t wait_ticks;      // bound on each wait for a ready flag (100 MHz ticks)
  moe::GemmKnobs knobs;     // test knobs of the GEMM launches (moe_ctx_set_debug)
  void* scratch;            // this device's address of `scratch`
};

namespace moe {

static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int make_geometry(const moe_shape_t* s, Geometry* g) {
  if (s == nullptr || g == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->R < 1 || s->R > MOE_MAX_RANKS || s->T < 1 || s->E < 1 || s->k < 1) return MOE_ERR_INVALID_ARG;
  if (s->E % s->R != 0) return MOE_ERR_INVALID_ARG;
  if (s->k > s->E || s->k > 16) return MOE_ERR_INVALID_ARG;
  if (s->r_self < 0 || s->r_self >= s->R) return MOE_ERR_INVALID_ARG;
  if ((s->gated != 0 && s->gated != 1) || (s->gate_kind != MOE_GATE_SOFTMAX && s->gate_kind != MOE_GATE_SIGMOID))
    return MOE_ERR_INVALID_ARG;
  if (s->mgb < 1) return MOE_ERR_INVALID_ARG;
  if (s->H < 256 || s->H % 256 != 0 || s->F < 128 || s->F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->tb_m != 16 && s->tb_m != 32 && s->tb_m != 64 && s->tb_m != 128 && s->tb_m != 256)
    return MOE_ERR_UNSUPPORTED;
  if (s->E > 512) return MOE_ERR_UNSUPPORTED;
  const int El = s->E / s->R;
  if (El > 256 || (int64_t)El * s->R > 2048) return MOE_ERR_UNSUPPORTED;
  const int64_t n_tok = (int64_t)s->R * s->T;
  if (n_tok * s->k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  g->R = s->R; g->T = s->T; g->H = s->H; g->F = s->F; g->E = s->E; g->k = s->k;
  g->r_self = s->r_self; g->gated = s->gated; g->gate_kind = s->gate_kind;
  g->tb_m = s->tb_m; g->mgb = s->mgb;
  g->El = El;
  g->chunks_per_rank = (int32_t)ceil_div64(s->T, kChunk);
  g->n_chunks = g->chunks_per_rank * s->R;
  const int64_t valid_max = n_tok * (s->k < El ? s->k : El);
  const int64_t m_pad_max = valid_max + (int64_t)El * s->R * (s->tb_m - 1);
  if (m_pad_max * (s->H > s->F ? s->H : s->F) >= (int64_t)1 << 40 || m_pad_max >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  g->rows = ceil_div64(m_pad_max, s->tb_m) * s->tb_m;
  g->max_bands = (int32_t)(g->rows / s->tb_m);
  g->tile_m = kTileM;
  g->m_pad_max = g->rows + g->tile_m;   // the last tile may read past the last row
  g->max_tiles = (int32_t)(ceil_div64(g->rows, g->tile_m) + El);
  // per-shape tile table: output projection 256 wide; first projection
  // 256-wide MFMA tiles (128 h columns when gated)
  g->bn2 = 256;
  g->tiles2 = s->H / g->bn2;
  if (s->gated) { g->bn1 = 256; g->bn1_out = 128; }
  else if (s->F % 256 == 0) { g->bn1 = 256; g->bn1_out = 256; }
  else { g->bn1 = 128; g->bn1_out = 128; }
  g->tiles1 = s->F / g->bn1_out;
  const int64_t flags = (int64_t)g->max_tiles * g->tiles2;
  if (flags >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  g->max_flags = (int32_t)flags;
  g->recv_rows_max = (int32_t)((int64_t)s->T * (s->k < El ? s->k : El));
  // the consumer addresses a segment's 16-byte words with 32-bit offsets, and
  // the copying roles read a segment (at most mgb bands) through a buffer
  // resource with 32-bit byte offsets
  if ((int64_t)g->recv_rows_max * (s->H / 8) >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)s->mgb * s->tb_m * s->H * 2 >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

WsLayout ws_layout(const Geometry& g) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t n_i32) {
    const size_t at = off;
    off += (n_i32 * 4 + 255) / 256 * 256;
    return at;
  };
  const size_t nce = (size_t)g.n_chunks * g.El, er = (size_t)g.El * g.R, mb = (size_t)g.max_bands;
  L.meta = take(META_WORDS);
  L.chunk_counts = take(nce);
  L.chunk_base = take(nce);
  L.group_row = take(er);
  L.expert_base = take(g.El + 1);
  L.recv_off = take(er);
  L.band_row0 = take(mb); L.band_expert = take(mb); L.band_dest = take(mb);
  L.band_recv0 = take(mb); L.band_valid = take(mb);
  L.seg_band0 = take(mb); L.seg_nbands = take(mb); L.seg_dest = take(mb);
  L.seg_src_row = take(mb); L.seg_dst_row = take(mb); L.seg_rows = take(mb);
  L.row_src = take((size_t)g.m_pad_max);
  L.recv_row = take((size_t)g.R * g.T * g.k);
  L.tile_ctr = take(kCtrWords);
  L.slot_valid = take(mb);
  L.seg_unit0 = take(mb);
  L.partial = take((size_t)kXcds * kTailSlots * g.tile_m * 256);
  const size_t mt = (size_t)g.max_tiles;
  L.tile_row0 = take(mt); L.tile_expert = take(mt); L.tile_rows = take(mt); L.tile_sched = take(mt);
  L.seg_tile0 = take(mb); L.seg_tile1 = take(mb);
  L.zero_row = take((size_t)g.H / 2);
  L.total = off;
  return L;
}

void plan_from_ws(const Geometry& g, void* ws, moe_plan_t* p) {
  const WsLayout L = ws_layout(g);
  char* b = static_cast<char*>(ws);
  auto at = [&](size_t o) { return reinterpret_cast<int32_t*>(b + o); };
  p->meta = at(L.meta);
  p->group_row = at(L.group_row);
  p->expert_base = at(L.expert_base);
  p->recv_off = at(L.recv_off);
  p->band_row0 = at(L.band_row0); p->band_expert = at(L.band_expert); p->band_dest = at(L.band_dest);
  p->band_recv0 = at(L.band_recv0); p->band_valid = at(L.band_valid);
  p->seg_band0 = at(L.seg_band0); p->seg_nbands = at(L.seg_nbands); p->seg_dest = at(L.seg_dest);
  p->seg_src_row = at(L.seg_src_row); p->seg_dst_row = at(L.seg_dst_row); p->seg_rows = at(L.seg_rows);
  p->row_src = at(L.row_src);
  p->recv_row = at(L.recv_row);
  p->chunk_base = at(L.chunk_base);
  p->chunk_counts = at(L.chunk_counts);
  p->tile_ctr = at(L.tile_ctr);
  p->slot_valid = at(L.slot_valid);
  p->seg_unit0 = at(L.seg_unit0);
  p->partial = reinterpret_cast<float*>(b + L.partial);
  p->tile_row0 = at(L.tile_row0); p->tile_expert = at(L.tile_expert); p->tile_rows = at(L.tile_rows);
  p->tile_sched = at(L.tile_sched); p->seg_tile0 = at(L.seg_tile0); p->seg_tile1 = at(L.seg_tile1);
}

uint16_t* zero_row_of(const Geometry& g, void* ws) {
  return reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + ws_layout(g).zero_row);
}

static inline bool ws_ok(const void* ws) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0;
}

static inline int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_error_string(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or tile configuration";
    case MOE_ERR_WORKSPACE: return "workspace pointer missing or not 256-byte aligned";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "device watchdog: a ready-flag wait exceeded its budget";
    case MOE_ERR_DEVICE: return "device-side consistency check failed";
    default: return "unknown error";
  }
}

int moe_query_sizes(const moe_shape_t* shape, moe_sizes_t* out) {
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  Geometry g;
  const int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  out->ws_bytes = ws_layout(g).total;
  out->m_pad_max = g.m_pad_max;
  out->max_bands = g.max_bands;
  out->max_flags = g.max_flags;
  out->recv_rows_max = g.recv_rows_max;
  out->bn_out = g.bn2;
  out->tile_m = g.tile_m;
  out->max_tiles = g.max_tiles;
  return MOE_OK;
}

int moe_plan_view(const moe_shape_t* shape, void* ws, moe_plan_t* out) {
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  Geometry g;
  const int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  plan_from_ws(g, ws, out);
  return MOE_OK;
}

int moe_ctx_create(moe_ctx_t** out) {
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe_ctx* c = new moe_ctx();
  c->timing = 0;
  c->timed = 0;
  c->trace = nullptr;
  c->trace_flags = 0;
  c->wait_ticks = moe::kDefaultWaitTicks;
  c->knobs = moe::GemmKnobs{0u, 0, moe::kDefaultTailWaitTicks};
  if (hipGetDevice(&c->device) != hipSuccess ||
      hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device) != hipSuccess) {
    delete c;
    return MOE_ERR_HIP;
  }
  const int src = scratch_address(c->device, &c->scratch);
  if (src != MOE_OK) {
    delete c;
    return src;
  }
  *out = c;
  return MOE_OK;
}

int moe_ctx_set_timing(moe_ctx_t* ctx, int enable) {
  if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
  if (enable && !ctx->timing) {
    for (int i = 0; i < 5; ++i)
      if (hipEventCreate(&ctx->tev[i]) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(ctx->tev[j]);
        return MOE_ERR_HIP;
      }
    ctx->timing = 1;
  } else if (!enable && ctx->timing) {
    for (int i = 0; i < 5; ++i) (void)hipEventDestroy(ctx->tev[i]);
    ctx->timing = 0;
  }
  ctx->timed = 0;
  return MOE_OK;
}

int moe_ctx_timings(moe_ctx_t* ctx, float* ms) {
  if (ctx == nullptr || ms == nullptr || !ctx->timing || !ctx->timed) return MOE_ERR_INVALID_ARG;
  if (hipEventSynchronize(ctx->tev[4]) != hipSuccess) return MOE_ERR_HIP;
  float t01, t12, t13, t04, t23;
  if (hipEventElapsedTime(&t01, ctx->tev[0], ctx->tev[1]) != hipSuccess ||
      hipEventElapsedTime(&t12, ctx->tev[1], ctx->tev[2]) != hipSuccess ||
      hipEventElapsedTime(&t13, ctx->tev[1], ctx->tev[3]) != hipSuccess ||
      hipEventElapsedTime(&t04, ctx->tev[0], ctx->tev[4]) != hipSuccess ||
      hipEventElapsedTime(&t23, ctx->tev[2], ctx->tev[3]) != hipSuccess)
    return MOE_ERR_HIP;
  ms[0] = t01;
  ms[1] = t12;
  ms[2] = t13;
  ms[3] = t04;
  ms[4] = t23 > 0.f ? t23 : 0.f;
  if (ctx->timed_mode == MOE_MODE_OVERLAP || ctx->timed_mode == MOE_MODE_ROLE_SWITCH) {
    // one launch holds both roles: the exposed transfer comes from its device
    // clock stamps (100 MHz) of the last tile's completion and the last copy's
    uint64_t st[2];
    if (hipMemcpy(st, ctx->timed_meta + META_T_PROD, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess)
      return MOE_ERR_HIP;
    // st[0] stays 0 when no workgroup ran a tile (an empty layout), st[1]
    // when nothing was copied
    ms[4] = st[0] != 0 && st[1] > st[0] ? (float)((double)(st[1] - st[0]) * 1e-5) : 0.f;
  }
  return MOE_OK;
}

int moe_ctx_set_trace(moe_ctx_t* ctx, const moe_shape_t* shape, uint64_t* trace, int64_t words) {
  if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
  if (trace == nullptr) {
    ctx->trace = nullptr;
    return MOE_OK;
  }
  Geometry g;
  const int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (words < 8 + (int64_t)g.max_flags + 3 * (int64_t)g.max_bands) return MOE_ERR_INVALID_ARG;
  ctx->trace = trace;
  ctx->trace_flags = g.max_flags;
  return MOE_OK;
}

int moe_ctx_destroy(moe_ctx_t* ctx) {
  if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
  const int rc = ctx->timing ? moe_ctx_set_timing(ctx, 0) : MOE_OK;
  delete ctx;
  return rc;
}

int moe_ctx_num_cus(const moe_ctx_t* ctx) { return ctx ? ctx->n_cu : MOE_ERR_INVALID_ARG; }

int moe_ctx_set_wait_limit(moe_ctx_t* ctx, uint64_t ticks) {
  if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
  ctx->wait_ticks = ticks == 0 ? moe::kDefaultWaitTicks : ticks;
  return MOE_OK;
}

int moe_ctx_set_debug(moe_ctx_t* ctx, uint32_t delay_seed, int32_t reverse_schedule, int64_t tail_wait_ticks) {
  if (ctx == nullptr || (reverse_schedule != 0 && reverse_schedule != 1)) return MOE_ERR_INVALID_ARG;
  ctx->knobs.delay_seed = delay_seed;
  ctx->knobs.reverse = reverse_schedule;
  ctx->knobs.tail_wait_ticks = tail_wait_ticks < 0 ? moe::kDefaultTailWaitTicks : (uint64_t)tail_wait_ticks;
  return MOE_OK;
}

int moe_route(const moe_shape_t* shape, const float* logits, int32_t* topk_ids, float* gates,
              int32_t* counts, void* ws, void* stream) {
  Geometry g;
  int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!logits || !topk_ids || !gates || !counts) return MOE_ERR_INVALID_ARG;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  moe_plan_t p;
  plan_from_ws(g, ws, &p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_rc(launch_route(g, logits, topk_ids, gates, p, st));
  if (rc != MOE_OK) return rc;
  return hip_rc(launch_count(g, topk_ids, counts, p, st));
}

int moe_permute(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_ids,
                const int32_t* counts, uint16_t* x_perm, void* ws, void* stream) {
  Geometry g;
  int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!topk_ids || !counts || (x_perm && !x)) return MOE_ERR_INVALID_ARG;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  moe_plan_t p;
  plan_from_ws(g, ws, &p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the plan also evaluates the CU-split model for this device (MOE_CONSUMER_AUTO)
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  const moe_calib_t calib = default_calib(n_cu);
  if ((rc = hip_rc(launch_plan(g, counts, topk_ids, p, zero_row_of(g, ws), calib, st))) != MOE_OK) return rc;
  return hip_rc(launch_gather(g, x, x_perm, p, st));
}

}  // extern "C"

// Both expert-phase entry points: `a` is x_perm (gathered = false) or x
// (gathered = true: the first projection reads packed row r from x row
// row_src[r], or the workspace's zero row for padding).
// use_scratch: the GEMMs' counters and K-split partials come from the
// library's static scratch instead of the workspace (moe_expert_forward_noalloc)
static int expert_forward(moe_ctx_t* ctx, const moe_shape_t* shape, const uint16_t* a, bool gathered,
                          const uint16_t* w1, const uint16_t* w3, const uint16_t* w2, void* ws,
                          uint16_t* h, uint16_t* y_perm, uint16_t* const* combine_buf, uint32_t* flags,
                          uint32_t epoch, int32_t n_consumer_cu, int32_t mode, void* stream,
                          bool use_scratch = false) {
  Geometry g;
  int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!ctx || !a || !w1 || !w2 || !h || !y_perm || !combine_buf) return MOE_ERR_INVALID_ARG;
  if ((g.gated != 0) != (w3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_MODE_OVERLAP && mode != MOE_MODE_SEQUENTIAL && mode != MOE_MODE_ROLE_SWITCH)
    return MOE_ERR_INVALID_ARG;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  BufPtrs bufs{};
  for (int s = 0; s < g.R; ++s) {
    if (s == g.r_self) continue;
    if (combine_buf[s] == nullptr) return MOE_ERR_INVALID_ARG;
    bufs.p[s] = combine_buf[s];
  }
  const bool auto_c = n_consumer_cu == MOE_CONSUMER_AUTO;
  if (mode == MOE_MODE_OVERLAP) {
    if (!flags || epoch == 0 ||
        (!auto_c && (n_consumer_cu < 1 || n_consumer_cu > 64 || n_consumer_cu >= ctx->n_cu)))
      return MOE_ERR_INVALID_ARG;
  } else if (mode == MOE_MODE_ROLE_SWITCH) {
    if (!flags || epoch == 0) return MOE_ERR_INVALID_ARG;
  } else if (!auto_c && (n_consumer_cu < 0 || n_consumer_cu > 64 || n_consumer_cu >= ctx->n_cu)) {
    return MOE_ERR_INVALID_ARG;
  }
  moe_plan_t p;
  plan_from_ws(g, ws, &p);
  hipStream_t ps = static_cast<hipStream_t>(stream);
  if (use_scratch) {
    // the largest partial tile either GEMM writes is tile_m x 256 fp32
    const size_t need = kScratchCtrBytes + (size_t)kXcds * kTailSlots * g.tile_m *
                                               (size_t)(g.bn1 > g.bn2 ? g.bn1 : g.bn2) * 4;
    if (need > kScratchBytes || ctx->scratch == nullptr) return MOE_ERR_UNSUPPORTED;
    p.tile_ctr = static_cast<int32_t*>(ctx->scratch);
    p.partial = reinterpret_cast<float*>(static_cast<char*>(ctx->scratch) + kScratchCtrBytes);
    // the array keeps the last call's counters: clear them first
    hipLaunchKernelGGL(k_clear_scratch_ctr, dim3(1), dim3(256), 0, ps, p.tile_ctr, (int)kCtrWords);
    if ((rc = hip_rc(hipGetLastError())) != MOE_OK) return rc;
  }
  const int ncu = ctx->n_cu;
  const bool tm = ctx->timing != 0;
  auto rec = [&](int i, hipStream_t st) { return tm ? hip_rc(hipEventRecord(ctx->tev[i], st)) : MOE_OK; };
  if ((rc = rec(0, ps)) != MOE_OK) return rc;
  if ((rc = hip_rc(launch_gemm1(g, a, gathered ? p.row_src : nullptr, gathered ? zero_row_of(g, ws) : nullptr,
                                w1, w3, h, p, mode == MOE_MODE_SEQUENTIAL ? nullptr : flags, ncu, ctx->knobs,
                                ps))) !=
      MOE_OK)
    return rc;
  if ((rc = rec(1, ps)) != MOE_OK) return rc;
  if (mode == MOE_MODE_SEQUENTIAL) {
    if ((rc = hip_rc(launch_gemm2(g, h, w2, y_perm, p, nullptr, 0, ctx->trace, ncu,
                                  auto_c ? 0 : ncu - n_consumer_cu, nullptr, 0, nullptr, ctx->wait_ticks,
                                  ctx->knobs, ps))) != MOE_OK)
      return rc;
    if ((rc = rec(2, ps)) != MOE_OK) return rc;
    if ((rc = hip_rc(launch_bulk_copy(g, y_perm, bufs, p, MOE_BULK_WG_PER_CU * ncu, ps))) != MOE_OK) return rc;
    if ((rc = rec(3, ps)) != MOE_OK) return rc;
    if ((rc = rec(4, ps)) != MOE_OK) return rc;
    ctx->timed = tm;
    ctx->timed_mode = mode;
    return MOE_OK;
  }
  if (mode == MOE_MODE_ROLE_SWITCH) {
    // one launch on every CU does both duties; the split is sized for all CUs
    if ((rc = hip_rc(launch_gemm2(g, h, w2, y_perm, p, flags, epoch, ctx->trace, ncu, ncu, &bufs, 0, nullptr,
                                  ctx->wait_ticks, ctx->knobs, ps))) != MOE_OK)
      return rc;
    if ((rc = rec(2, ps)) != MOE_OK) return rc;
    if ((rc = rec(3, ps)) != MOE_OK) return rc;
    if ((rc = rec(4, ps)) != MOE_OK) return rc;
    ctx->timed_meta = p.meta;
    ctx->timed = tm;
    ctx->timed_mode = mode;
    return MOE_OK;
  }
  // CU partition: one launch on every CU, workgroups [0, c) the consumer
  if ((rc = hip_rc(launch_gemm2(g, h, w2, y_perm, p, flags, epoch, ctx->trace, ncu,
                                auto_c ? 0 : ncu - n_consumer_cu, nullptr, auto_c ? -1 : n_consumer_cu, &bufs,
                                ctx->wait_ticks, ctx->knobs, ps))) != MOE_OK)
    return rc;
  if ((rc = rec(2, ps)) != MOE_OK) return rc;
  if ((rc = rec(3, ps)) != MOE_OK) return rc;
  if ((rc = rec(4, ps)) != MOE_OK) return rc;
  ctx->timed_meta = p.meta;
  ctx->timed = tm;
  ctx->timed_mode = mode;
  return MOE_OK;
}

extern "C" {

int moe_expert_forward_overlap(moe_ctx_t* ctx, const moe_shape_t* shape, const uint16_t* x_perm,
                               const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                               void* ws, uint16_t* h, uint16_t* y_perm,
                               uint16_t* const* combine_buf, uint32_t* flags, uint32_t epoch,
                               int32_t n_consumer_cu, int32_t mode, void* stream) {
  return expert_forward(ctx, shape, x_perm, false, w1, w3, w2, ws, h, y_perm, combine_buf, flags, epoch,
                        n_consumer_cu, mode, stream);
}

int moe_expert_forward_gathered(moe_ctx_t* ctx, const moe_shape_t* shape, const uint16_t* x,
                                const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                                void* ws, uint16_t* h, uint16_t* y_perm,
                                uint16_t* const* combine_buf, uint32_t* flags, uint32_t epoch,
                                int32_t n_consumer_cu, int32_t mode, void* stream) {
  return expert_forward(ctx, shape, x, true, w1, w3, w2, ws, h, y_perm, combine_buf, flags, epoch,
                        n_consumer_cu, mode, stream);
}

int moe_expert_forward_noalloc(moe_ctx_t* ctx, const moe_shape_t* shape, const uint16_t* x_perm,
                               const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                               void* ws, uint16_t* h, uint16_t* y_perm,
                               uint16_t* const* combine_buf, uint32_t* flags, uint32_t epoch,
                               int32_t n_consumer_cu, int32_t mode, void* stream) {
  return expert_forward(ctx, shape, x_perm, false, w1, w3, w2, ws, h, y_perm, combine_buf, flags, epoch,
                        n_consumer_cu, mode, stream, true);
}

int moe_combine(const moe_shape_t* shape, uint16_t* const* combine_buf, const uint16_t* y_perm,
                const float* gates, void* ws, uint16_t* y_share, void* stream) {
  Geometry g;
  int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!combine_buf || !y_perm || !gates || !y_share) return MOE_ERR_INVALID_ARG;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  BufPtrs bufs{};
  for (int s = 0; s < g.R; ++s) {
    if (s == g.r_self) continue;
    if (combine_buf[s] == nullptr) return MOE_ERR_INVALID_ARG;
    bufs.p[s] = combine_buf[s];
  }
  moe_plan_t p;
  plan_from_ws(g, ws, &p);
  return hip_rc(launch_combine(g, bufs, y_perm, gates, p, y_share, static_cast<hipStream_t>(stream)));
}

int moe_read_status(const moe_shape_t* shape, void* ws, int32_t* status, void* stream) {
  Geometry g;
  const int rc = make_geometry(shape, &g);
  if (rc != MOE_OK) return rc;
  if (!status) return MOE_ERR_INVALID_ARG;
  if (!ws_ok(ws)) return MOE_ERR_WORKSPACE;
  moe_plan_t p;
  plan_from_ws(g, ws, &p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(status, p.meta + META_STATUS, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
  return *status;
}

}  // extern "C"
