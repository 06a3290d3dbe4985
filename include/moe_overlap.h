/*
 * moe_overlap.h -- C ABI of the MI355X (gfx950) library for one
 * expert-parallel rank's MoE-layer share with tile-signalled combine overlap.
 *
 * Method: "Fine-grained Computation-Communication Overlap via Tile-level
 * Signaling and Scheduling for Mixture-of-Experts" (arXiv 2607.19539),
 * cited as [TLS] below; the per-layer producer/consumer split follows the
 * cost-model idea in the abstract of "Weave: Fine-Grained Dynamic SM
 * Scheduling in an MoE Megakernel for Compute-Communication Overlap"
 * (arXiv 2609.21483), cited as [Weave].
 *
 * One call sequence computes rank r_self's share of an MoE layer
 * ([TLS] sec. 2.1, steps 1-5, with the two all-to-alls modelled on one GPU):
 *
 *   moe_route       top-k routing, gates, per-(local expert, source rank) counts
 *   moe_plan_partition (optional, host) consumer CU count / segment size
 *   moe_permute     remote-owner-aligned row layout, band schedule, combine
 *                   plan, transfer segments, gather of the routed rows
 *   moe_expert_forward_overlap
 *                   expert FFN as a persistent grouped GEMM; its output
 *                   projection raises one ready flag per tile while the
 *                   same launch's consumer workgroups on a few CUs (or,
 *                   role switching, the producer's own workgroups between
 *                   tiles) copy each ready segment into its source rank's
 *                   combine buffer
 *   moe_expert_forward_gathered
 *                   the same, its first projection reading the routed rows
 *                   straight from x (the gather fused into the tile loads)
 *   moe_combine     gate-weighted reduction of the returned rows
 *
 * Conventions
 *  - Every tensor argument is a DEVICE pointer allocated and owned by the
 *    caller; the library never allocates device memory on these paths and
 *    never frees caller memory. bf16 tensors are passed as uint16_t bit
 *    patterns; all matrices are row-major and densely packed.
 *  - Every call except moe_query_sizes, moe_plan_partition, moe_error_string
 *    and moe_ctx_* only enqueues work on the given HIP stream (passed as
 *    void*, NULL = the default stream) and returns without synchronising.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code. Argument and
 *    shape errors are detected on the host before any HIP call.
 *  - No global state: everything persistent lives in caller memory (the
 *    workspace) or in a moe_ctx_t.
 */
#ifndef MOE_OVERLAP_H
#define MOE_OVERLAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, bad size, inconsistent shape  */
#define MOE_ERR_UNSUPPORTED (-2)  /* shape/tile outside the compiled tile table  */
#define MOE_ERR_WORKSPACE   (-3)  /* workspace pointer misaligned                */
#define MOE_ERR_HIP         (-4)  /* a HIP runtime call failed                   */
#define MOE_ERR_TIMEOUT     (-5)  /* device watchdog: a flag wait exceeded budget */
#define MOE_ERR_DEVICE      (-6)  /* device-side consistency check failed         */

#define MOE_MAX_RANKS 16          /* R limit: combine buffer pointers go by value */

enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 };
enum { MOE_MODE_OVERLAP = 0, MOE_MODE_SEQUENTIAL = 1, MOE_MODE_ROLE_SWITCH = 2 };
/* n_consumer_cu of the expert forward: the plan's own choice (see moe_permute) */
#define MOE_CONSUMER_AUTO (-1)

/* Problem shape of one rank's share ([TLS] sec. 3.2, Algorithm 1 inputs).
 *  R        simulated ranks (1..MOE_MAX_RANKS)
 *  T        tokens per rank (>= 1)
 *  H        hidden size (multiple of 256)
 *  F        expert FFN width (multiple of 128)
 *  E        experts in total; E % R == 0; rank r owns experts [r*E/R, (r+1)*E/R)
 *  k        top-k, 1 <= k <= min(E, 16)
 *  r_self   the rank whose share is computed, 0 <= r_self < R
 *  gated    1: y = (SiLU(x W1^T) * (x W3^T)) W2^T;  0: y = SiLU(x W1^T) W2^T
 *  gate_kind MOE_GATE_SOFTMAX: softmax over the k selected logits;
 *           MOE_GATE_SIGMOID: sigmoid of the k selected logits, normalised to sum 1
 *  tb_m     row-band height ([TLS] sec. 3.2.1): the padding unit of the owner
 *           groups and the transfer unit of the combine plan: 16, 32, 64,
 *           128 or 256. The GEMMs run tiles of moe_sizes_t.tile_m (256) rows
 *           over each expert's tb_m-aligned rows, so the band can be smaller
 *           than the compute tile (and, at 16, than one 32-row MFMA block).
 *  mgb      row bands per middle transfer segment ([TLS] sec. 3.3.2, Fig. 3(b)), >= 1,
 *           with mgb * tb_m * H * 2 < 2^31 (a segment below 2 GiB)
 */
typedef struct {
  int32_t R, T, H, F, E, k, r_self;
  int32_t gated, gate_kind;
  int32_t tb_m, mgb;
} moe_shape_t;

/* Buffer sizes for a shape. Packed rows are bounded by
 * rows = min(R*T*k, R*T*E/R) + (E/R)*R*(tb_m-1) rounded up to tb_m (each remote
 * owner group is padded by < tb_m rows and each expert's rows are placed
 * tb_m-aligned); the row buffers carry tile_m more rows, which the last GEMM
 * tile of the last expert may read (never write). */
typedef struct {
  size_t  ws_bytes;       /* workspace bytes (256-byte aligned pointer required) */
  int64_t m_pad_max;      /* rows to allocate for x_perm [.,H], h [.,F], y_perm [.,H]:
                             rows + tile_m */
  int32_t max_bands;      /* = rows / tb_m */
  int32_t max_flags;      /* uint32 ready flags the overlapped forward may write
                             (max_tiles * H / bn_out) */
  int32_t recv_rows_max;  /* rows to allocate per combine buffer: T*min(k, E/R) */
  int32_t bn_out;         /* column-tile width of the output projection */
  int32_t tile_m;         /* GEMM row-tile height (256) */
  int32_t max_tiles;      /* GEMM row tiles at most: ceil(rows / tile_m) + E/R */
} moe_sizes_t;

/* Read-only device views into a workspace after moe_permute (for inspection
 * and tests). Arrays indexed by band / segment are in schedule order. */
typedef struct {
  int32_t* meta;          /* [0]=m_pad [1]=n_bands [2]=n_remote_bands [3]=n_segments
                             [4]=device status (0 or MOE_ERR_*) [5]=64 KiB copy units
                             [6]=GEMM row tiles [7]=tiles holding a remote band
                             [8]=consumer CUs chosen by the plan (MOE_CONSUMER_AUTO)
                             [20..21]=its predicted time in seconds (a double; -1 if
                             the device evaluation fell back to c_min)
                             [16..19]=internal clock stamps of the overlapped forward
                             [22]=internal: arrivals of the routing histogram */
  int32_t* group_row;     /* [E_l*R] first packed row of group (e, s)                */
  int32_t* expert_base;   /* [E_l+1] first packed row of expert e, tb_m-aligned      */
  int32_t* recv_off;      /* [R*E_l] first row of (e, s) in rank s's combine buffer */
  int32_t* band_row0;     /* [max_bands] first packed row of the band                */
  int32_t* band_expert;   /* [max_bands] local expert                                 */
  int32_t* band_dest;     /* [max_bands] owner rank (r_self for local bands)          */
  int32_t* band_recv0;    /* [max_bands] first combine-buffer row, -1 if local        */
  int32_t* band_valid;    /* [max_bands] non-padding rows                             */
  int32_t* seg_band0;     /* [max_bands] first band (schedule index) of the segment   */
  int32_t* seg_nbands;    /* [max_bands]                                              */
  int32_t* seg_dest;      /* [max_bands]                                              */
  int32_t* seg_src_row;   /* [max_bands] first y_perm row                             */
  int32_t* seg_dst_row;   /* [max_bands] first combine-buffer row                     */
  int32_t* seg_rows;      /* [max_bands] valid rows copied                            */
  int32_t* row_src;       /* [m_pad_max] token s*T+t of each packed row, -1 = zero row */
  int32_t* recv_row;      /* [R*T*k] combine-buffer row (s != r_self) or y_perm row
                             (s == r_self) of slot j of token g; -1 if not local      */
  int32_t* chunk_base;    /* [n_chunks*E_l] internal: per-chunk row offsets           */
  int32_t* chunk_counts;  /* [n_chunks*E_l] internal: per-chunk local counts          */
  int32_t* tile_ctr;      /* internal: per-XCD tile queue counters of the two GEMMs   */
  int32_t* slot_valid;    /* [max_bands] valid rows of the band starting at row tb_m*i */
  int32_t* seg_unit0;     /* [max_bands] internal: first 64 KiB copy unit of each segment */
  int32_t* tile_row0;     /* [max_tiles] GEMM row tile i (layout order: experts by id,
                             tile_m rows each from the expert's base): first packed row */
  int32_t* tile_expert;   /* [max_tiles] its local expert                               */
  int32_t* tile_rows;     /* [max_tiles] its rows inside the expert's tb_m-aligned rows
                             (tile_m except for an expert's last tile); rows past these
                             are computed from the next rows but never stored            */
  int32_t* tile_sched;    /* [max_tiles] tile at each position of the GEMM schedule:
                             tiles holding any remote band first (experts in the band
                             schedule's order), then the others by expert id            */
  int32_t* seg_tile0;     /* [max_bands] first tile covering the segment's bands       */
  int32_t* seg_tile1;     /* [max_bands] last tile covering the segment's bands        */
  float*   partial;       /* internal: fp32 partial tiles of the GEMMs' K-split tail tiles */
} moe_plan_t;

/* Calibration of the partition cost model (measured on the device). */
typedef struct {
  double gemm_flops_per_cu;   /* sustained bf16 FLOP/s of one producer CU, large M */
  double gemm_m_half;         /* rows per expert at which GEMM efficiency halves
                                 (0: every expert at the full rate)                 */
  double copy_bw_per_cu;      /* b: bytes/s one consumer CU moves beside the GEMM   */
  double copy_bw_max;         /* B: bytes/s the copy saturates at; c CUs move
                                 c b / (1 + c b / B)                                */
  double seg_latency_s;       /* fixed cost of the copy's last batch, seconds       */
  int32_t n_cu;               /* CUs on the device (256 on MI355X)                  */
  int32_t c_min, c_max;       /* consumer CU range considered                       */
  int32_t c_step;             /* candidates c_min, c_min + c_step, ...: a multiple of
                                 the XCD count (8) keeps both kernels' workgroups
                                 spread evenly over the XCDs                        */
} moe_calib_t;

typedef struct moe_ctx moe_ctx_t;

/* Human-readable name of an MOE_* code (static string, never NULL). */
const char* moe_error_string(int code);

/* Validates the shape and reports buffer sizes. Host only; no HIP call. */
int moe_query_sizes(const moe_shape_t* shape, moe_sizes_t* out);

/* Fills device views into a workspace of ws_bytes at ws. Host only. */
int moe_plan_view(const moe_shape_t* shape, void* ws, moe_plan_t* out);

/* Creates a context for the current HIP device: its CU count (the grids of
 * the expert forward) and, once enabled, timing events. Returns MOE_OK and
 * sets *out, or MOE_ERR_HIP. Destroy with moe_ctx_destroy. */
int moe_ctx_create(moe_ctx_t** out);
int moe_ctx_destroy(moe_ctx_t* ctx);
int moe_ctx_num_cus(const moe_ctx_t* ctx);

/* Bound on every wait of a copying role for the ready flags of a segment's
 * row tiles (the consumer of the CU-partition overlap, the copy duty of role
 * switching), in ticks of the 100 MHz constant clock; 0 restores the default
 * of 2 s. A wait that runs out sets the device status word (moe_read_status)
 * to MOE_ERR_TIMEOUT, and the waiting workgroups stop copying and exit; the
 * producer's tiles, and so y_perm, are unaffected, and the next moe_permute
 * clears the status. Applies to later moe_expert_forward_* calls on ctx.
 * A flag can only stay unset if the producer never reaches its tile (for
 * instance a preempted or failed launch); a tiny bound forces the error path
 * from the host. Returns MOE_ERR_INVALID_ARG for a NULL ctx. */
int moe_ctx_set_wait_limit(moe_ctx_t* ctx, uint64_t ticks);

/* Test knobs of later moe_expert_forward_* calls on ctx. They change only
 * when work happens, never the results, so outputs stay bit-identical to a
 * call without them (the race tests rely on that):
 *   delay_seed       nonzero: each GEMM work item sleeps a pseudo-random
 *                    0..23 x ~3.4 us, drawn from (seed, tile, chunk), before
 *                    its results are stored and flagged
 *   reverse_schedule 1: every GEMM tile queue runs its whole tiles in reverse
 *                    schedule order (the rank's own rows first, remote rows
 *                    last; the K-split tail tiles stay the same tiles), 0: as
 *                    scheduled ([TLS] sec. 3.2.2)
 *   tail_wait_ticks  bound on how long a K-chunk of one of the output
 *                    projection's split tail tiles waits for the tile's other
 *                    chunks, in 100 MHz ticks (< 0: the default of 1 ms); a
 *                    chunk that gives up leaves its share of the tile to the
 *                    chunk that arrives last, so 0 makes the last chunk of
 *                    every split tile reduce the whole tile
 * Returns MOE_ERR_INVALID_ARG for a NULL ctx or reverse_schedule not 0/1. */
int moe_ctx_set_debug(moe_ctx_t* ctx, uint32_t delay_seed, int32_t reverse_schedule, int64_t tail_wait_ticks);

/* Phase timing of moe_expert_forward_overlap with HIP events recorded on the
 * streams the kernels run on (off by default; enabling creates 5 events).
 * moe_ctx_timings waits for the last timed call and writes, in ms:
 *   ms[0] first projection (all CUs)
 *   ms[1] output projection launch (OVERLAP: producer and consumer roles;
 *         ROLE_SWITCH: with the copy)
 *   ms[2] from the output projection's start to the end of the transfer
 *         (SEQUENTIAL: to the end of the bulk copy)
 *   ms[3] whole call
 *   ms[4] exposed transfer: OVERLAP and ROLE_SWITCH, the completion of the
 *         last copy minus the completion of the last tile of the output
 *         projection (>= 0; 0 when nothing is copied), from device clock
 *         stamps of the same launch; SEQUENTIAL, the bulk copy's duration
 * Returns MOE_ERR_INVALID_ARG if timing is off or nothing was timed. */
int moe_ctx_set_timing(moe_ctx_t* ctx, int enable);
int moe_ctx_timings(moe_ctx_t* ctx, float* ms);

/* Device timeline of the overlapped expert phase (off when trace is NULL).
 * trace: caller device buffer of uint64 words, stamps of the 100 MHz constant
 * clock (wall_clock64), written by later moe_expert_forward_overlap calls:
 *   [0]                          output projection start (workgroup 0)
 *   [1]                          consumer start (workgroup 0)
 *   [8 + t]                      output-projection tile t stored and flagged
 *   [8 + max_flags + 3 s + 0/1/2] consumer workgroup 0, segment s: wait begins,
 *                                all its flags seen, its share of the copy done
 * words >= 8 + max_flags + 3 * max_bands (moe_sizes_t), else MOE_ERR_INVALID_ARG. */
int moe_ctx_set_trace(moe_ctx_t* ctx, const moe_shape_t* shape, uint64_t* trace, int64_t words);

/* Step 1, routing ([TLS] sec. 2.1 step 1). Per token g of R*T (g = s*T + t):
 * the k experts with the highest logits, highest first, equal logits to the
 * lower expert id; gates per gate_kind (they sum to 1).
 *   logits   [R*T, E] fp32 (in)
 *   topk_ids [R*T, k] int32 global expert ids (out)
 *   gates    [R*T, k] fp32 (out)
 *   counts   [E_l, R] int32 (out): count[e][s] = slots of rank s's tokens
 *            routed to local expert r_self*E_l + e (the rows the dispatch delivers)
 *   ws       workspace (per-chunk counts are left there for moe_permute) */
int moe_route(const moe_shape_t* shape, const float* logits, int32_t* topk_ids,
              float* gates, int32_t* counts, void* ws, void* stream);

/* Steps 3-4: remote-owner-aligned row layout, remote-first band schedule and
 * combine plan ([TLS] sec. 3.2.1-3.2.3, Algorithm 1), transfer segments
 * ([TLS] sec. 3.3.2, Fig. 3(b)), and the gather of the routed rows (the
 * dispatch, modelled locally).
 *   x       [R, T, H] bf16: every rank's tokens (in)
 *   topk_ids, counts: from moe_route (in)
 *   x_perm  [m_pad_max, H] bf16 (out): row i = x of token row_src[i]; zero
 *           rows for owner-boundary padding and between experts. Rows beyond
 *           m_pad are not written.
 *           NULL: no row is copied; the plan and the indexes (row_src with -1
 *           for every padding row, recv_row) are built as usual, for
 *           moe_expert_forward_gathered. x may then be NULL too.
 *   ws      workspace: plan arrays written (see moe_plan_t).
 * The plan kernel also evaluates the CU-split model of moe_plan_partition
 * (calib = NULL, with n_cu = the current device's CU count) on the device,
 * from this plan's row tiles and segments, and leaves c in meta[8] for
 * n_consumer_cu = MOE_CONSUMER_AUTO: the same c and predicted time as
 * moe_plan_partition returns for these counts when shape->mgb is the mgb it
 * returns. Plans past its table bounds (2048 row tiles, 2048 segments, 2048
 * producer waves over the candidates) take c_min. */
int moe_permute(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_ids,
                const int32_t* counts, uint16_t* x_perm, void* ws, void* stream);

/* Picks the consumer CU count c (and segment size) for one layer from the
 * routing counts ([Weave] abstract: split compute/communication workers to
 * match the layer's communication/computation ratio; [TLS] sec. 4.3.4 on the
 * cost of a wrong split). Host-only pure function.
 *   counts_host [E_l, R] int32 (host memory)
 *   calib       NULL = built-in MI355X defaults
 *   n_consumer_cu (out) c in {c_min, c_min + c_step, ...} <= c_max
 *               (defaults 8, 16, ..., 48)
 *   mgb         (out, may be NULL) bands per middle segment
 *   predicted_s (out, may be NULL) model time of the overlapped expert phase */
int moe_plan_partition(const moe_shape_t* shape, const int32_t* counts_host,
                       const moe_calib_t* calib, int32_t* n_consumer_cu, int32_t* mgb,
                       double* predicted_s);

/* Step 3+4: expert FFN + combine transfer ([TLS] sec. 3.3).
 *   x_perm   [m_pad_max, H] bf16 from moe_permute
 *   w1, w3   [E_l, F, H] bf16 (nn.Linear [out, in]); w3 NULL iff !gated
 *   w2       [E_l, H, F] bf16
 *   h        [m_pad_max, F] bf16 scratch (the activated first projection)
 *   y_perm   [m_pad_max, H] bf16 (out): expert outputs in packed row order
 *   combine_buf host array of R device pointers; combine_buf[s] for s != r_self
 *            is [recv_rows_max, H] bf16 (out): rows returned to rank s;
 *            combine_buf[r_self] is ignored (may be NULL)
 *   flags    [max_flags] uint32 (OVERLAP, ROLE_SWITCH; may be NULL in
 *            SEQUENTIAL): the first projection clears them, the output
 *            projection sets flags[t] = epoch once tile t is stored
 *   epoch    nonzero. Every call starts from cleared flags, so repeated
 *            calls may reuse one epoch (a captured call replayed from a HIP
 *            graph does)
 *   n_consumer_cu  c: OVERLAP 1..64, SEQUENTIAL 0..64, and < device CUs; or
 *            MOE_CONSUMER_AUTO (OVERLAP, SEQUENTIAL): the c the preceding
 *            moe_permute chose on the device, with no host round trip. The
 *            output projection splits its tail tiles along K for CUs - c
 *            producers in both modes, so OVERLAP and SEQUENTIAL calls with the
 *            same c compute bit-identical results (different c may differ in
 *            the last bits of the split tiles, from the fp32 summation order)
 *   mode     MOE_MODE_OVERLAP: first projection on all CUs; then one launch
 *            of the output projection on every CU whose first c workgroups
 *            (one per CU, c/8 per XCD) are the consumer, copying every segment
 *            once all its tiles are flagged, while the others run the tiles as
 *            persistent producers raising a flag per tile (one stream: the
 *            CU split comes from the roles of one grid, not from two kernels).
 *            A consumer workgroup whose share of the copy is done takes
 *            tiles still queued, as a producer.
 *            MOE_MODE_SEQUENTIAL (baseline, [TLS] sec. 4.1.3): both projections
 *            on all CUs, then one bulk copy of all remote rows on all CUs.
 *            MOE_MODE_ROLE_SWITCH: both projections on all CUs, the output
 *            projection's workgroups doing the consumer's work as well: before
 *            each tile a workgroup claims the next 64 KiB copy units of the
 *            remote segments (schedule order, up to 8 per claim and at most
 *            an even share of those left over 64 workgroups, one
 *            fetch-and-add) once the segment holding them has all its tiles
 *            flagged, and copies them; a claim stays with its workgroup until
 *            copied. Once the tiles run out the workgroups claim and copy the
 *            rest (each wait bounded like the consumer's). No CU is reserved; c is
 *            ignored and the K-split is sized for all CUs (the same bits as
 *            SEQUENTIAL with c = 0). The per-layer worker split of [Weave]
 *            taken to its temporal end.
 *   stream   every mode runs on this one stream: its work is ordered after
 *            prior work on it and completes before later work on it
 * Calls that overlap in time on the same flags/workspace race. */
int moe_expert_forward_overlap(moe_ctx_t* ctx, const moe_shape_t* shape,
                               const uint16_t* x_perm, const uint16_t* w1,
                               const uint16_t* w3, const uint16_t* w2, void* ws,
                               uint16_t* h, uint16_t* y_perm, uint16_t* const* combine_buf,
                               uint32_t* flags, uint32_t epoch, int32_t n_consumer_cu,
                               int32_t mode, void* stream);

/* moe_expert_forward_overlap with the gather fused into the first
 * projection (the dispatch side of [TLS] sec. 2.1 steps 2-3): instead of
 * x_perm it takes x [R, T, H] bf16 (every rank's tokens, as given to
 * moe_permute) and the first projection's tile loads read packed row r
 * straight from x row row_src[r] of the workspace's plan (a zero row for
 * padding), so x_perm is neither written nor read. Requires a preceding
 * moe_permute on this workspace (x_perm may be NULL there). Every other
 * argument, mode and output is as in moe_expert_forward_overlap, and h,
 * y_perm and the combine buffers are bit-identical to it for the same plan,
 * mode and n_consumer_cu. */
int moe_expert_forward_gathered(moe_ctx_t* ctx, const moe_shape_t* shape,
                                const uint16_t* x, const uint16_t* w1,
                                const uint16_t* w3, const uint16_t* w2, void* ws,
                                uint16_t* h, uint16_t* y_perm, uint16_t* const* combine_buf,
                                uint32_t* flags, uint32_t epoch, int32_t n_consumer_cu,
                                int32_t mode, void* stream);

/* moe_expert_forward_overlap for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, modes and results (bit-identical to
 * moe_expert_forward_overlap for the same plan, mode and n_consumer_cu), but
 * the GEMM launches' scratch, i.e. their tile-queue, tail and copy counters
 * and the fp32 partial tiles of their K-split tail tiles, lives in one
 * static device array of the library (62 MiB + 4 KiB, held by every GPU the
 * library runs on until the process ends; its address is looked up once per
 * device by moe_ctx_create) instead of the workspace. The workspace still
 * carries the plan of the preceding moe_permute (its counter and partial
 * sections are left untouched). The call allocates nothing: it clears the
 * array's counters with a kernel on `stream`, then launches as
 * moe_expert_forward_overlap does. Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU race (as calls sharing a
 * workspace do). Returns MOE_ERR_UNSUPPORTED if a shape needed more scratch
 * than the array holds (none does: the largest partial tile is 256 x 256),
 * else as moe_expert_forward_overlap. */
int moe_expert_forward_noalloc(moe_ctx_t* ctx, const moe_shape_t* shape,
                               const uint16_t* x_perm, const uint16_t* w1,
                               const uint16_t* w3, const uint16_t* w2, void* ws,
                               uint16_t* h, uint16_t* y_perm, uint16_t* const* combine_buf,
                               uint32_t* flags, uint32_t epoch, int32_t n_consumer_cu,
                               int32_t mode, void* stream);

/* Step 5, weighted reduction ([TLS] sec. 2.1 step 5): for every token (s, t),
 * y_share[s, t] = sum over slots j ascending whose expert is local of
 * gates[s*T+t, j] * row, with row = combine_buf[s][recv_row] for s != r_self
 * and y_perm[recv_row] for s == r_self; fp32 accumulation, bf16 (RNE) out;
 * zero when no slot is local.
 *   combine_buf host array of R device pointers (as above)
 *   y_perm   [m_pad_max, H] bf16, gates [R*T, k] fp32
 *   y_share  [R, T, H] bf16 (out) */
int moe_combine(const moe_shape_t* shape, uint16_t* const* combine_buf,
                const uint16_t* y_perm, const float* gates, void* ws,
                uint16_t* y_share, void* stream);

/* Copies the device status word of the workspace to *status (host) and
 * synchronises the stream. Returns *status (MOE_OK, MOE_ERR_TIMEOUT, ...)
 * or MOE_ERR_HIP. MOE_ERR_TIMEOUT: a copying role's bounded wait for ready
 * flags ran out (moe_ctx_set_wait_limit); the combine buffers of that call
 * are then incomplete (y_perm is complete: no GEMM work item ever waits
 * without bound for another workgroup, so y_perm never depends on every
 * workgroup of a launch being resident at once). moe_permute clears it. */
int moe_read_status(const moe_shape_t* shape, void* ws, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OVERLAP_H */
