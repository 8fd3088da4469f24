/*
 * moe_overlap.h - C ABI of the MI355X (gfx950) MoE expert-compute-plus-return path.
 *
 * The method: "Fine-grained Computation-Communication Overlap via Tile-level Signaling and Scheduling for
 * Mixture-of-Experts" (Cui, Wingkvist, Ericsson; arXiv 2607.19539), as described on its review page.
 * An expert-parallel rank computes the expert FFN for every row routed to its local experts and returns
 * each output row to the rank that owns the token.  Rows are laid out grouped by (local expert, owner rank)
 * and padded to the tile height, so every output tile has one owner ("What carries the argument"; referee
 * major comment 1, section 4.5 / Algorithm 1).  A persistent grouped GEMM (the producer) publishes a
 * readiness flag per output tile while a persistent consumer on a small CU partition forwards finished
 * row-band segments to their owners ("The pith"; "Core claim").  Here all R owner ranks are R receive
 * buffers in the local HBM of one GPU: the consumer's transfers are device-memory copies.
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are device memory; everything else is host memory.  The caller owns every
 *    buffer; the library allocates no device memory and creates no streams, except three copy streams (default
 *    priority) per device that the DMA return mode of moe_expert_ffn_overlap creates on first use.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call is asynchronous on it.
 *  - Return values are moe_status codes for synchronous (host-side) checks: MOE_EINVAL for a bad shape,
 *    a null pointer or an unsupported size, MOE_EHIP when a HIP call or launch fails.  moe_last_error()
 *    gives a message.  Errors found on the device (an invalid token id, capacity overflow, a wait in the
 *    FFN launch that ran out of its spin budget) are written to the layout's device status word; read it
 *    with moe_read_status().  Kernels that follow a failed one see the nonzero status and do nothing.
 *  - Not thread-safe for one moe_layout; calls that share a layout or flag array must be ordered.
 *  - Matrices are row-major.  Weights follow the (out, in) convention of a linear layer.
 *  - Element type: MOE_BF16 (activations, weights, hidden h, outputs in bf16, fp32 accumulation) or
 *    MOE_F32 (everything fp32).  topk weights are always fp32, ids int32.
 */
#ifndef MOE_OVERLAP_H
#define MOE_OVERLAP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_OK = 0, MOE_EINVAL = -1, MOE_ECAPACITY = -2, MOE_EHIP = -3, MOE_ETIMEOUT = -4 } moe_status;
typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

#define MOE_MAX_OWNERS 16      /* R <= 16 owner ranks */
#define MOE_MAX_LOCAL_EXPERTS 64
#define MOE_SEG_FIELDS 8       /* int32 fields of one segment descriptor, see moe_layout.seg_desc */

/* Problem shape.  Tokens are owner-major: token row r*tokens_per_owner + t belongs to owner rank r.
 * Local experts are global ids [self_rank*num_local_experts, (self_rank+1)*num_local_experts). */
typedef struct {
  int32_t R;                  /* owner ranks, 1..MOE_MAX_OWNERS */
  int32_t tokens_per_owner;   /* T_o >= 0; T = R*T_o */
  int32_t num_global_experts; /* G >= 1 */
  int32_t num_local_experts;  /* E_l, 1..MOE_MAX_LOCAL_EXPERTS, G % E_l == 0 */
  int32_t top_k;              /* k, 1..min(G, 16) */
  int32_t self_rank;          /* this rank, 0 <= self_rank < G/E_l and < R */
  int32_t d;                  /* hidden size, multiple of 64 */
  int32_t f;                  /* FFN width, multiple of 64 */
  int32_t tile_m;             /* layout tile height M (rows per band), multiple of 16, <= 256 */
  int32_t seg_bands;          /* mgb: bands per transfer segment, >= 1 */
  int32_t dtype;              /* moe_dtype */
} moe_shape;

/* Layout and its metadata (all device pointers into one caller workspace, see moe_layout_bind).
 * Group g = e*R + r is the rows of owner r routed to local expert e, n_{e,r} rows, padded to
 * P = ceil(n/M)*M.  Band (tile) b covers padded rows [b*M, (b+1)*M). */
typedef struct {
  int32_t* counts;       /* [E_l*R]  n_{e,r} */
  int32_t* padded_off;   /* [E_l*R]  first padded row of group g: exclusive prefix of P in g order */
  int32_t* recv_off;     /* [E_l*R]  first row of group g in owner r's receive buffer: sum_{e'<e} n_{e',r} */
  int32_t* tile_owner;   /* [cap_tiles] owner of band b */
  int32_t* tile_expert;  /* [cap_tiles] local expert of band b */
  int32_t* tile_valid;   /* [cap_tiles] real rows in band b (1..M) */
  int32_t* tile_order;   /* [cap_tiles] bands in remote-first order: groups by (owner == self, -P, e, r),
                            bands ascending inside a group */
  int32_t* seg_desc;     /* [cap_tiles][MOE_SEG_FIELDS] transfer segments in tile_order order, each up to
                            seg_bands bands of one group: {owner, expert, first_band, n_bands, src_row,
                            dst_row, rows, group}; rows counts real rows only */
  int32_t* row_src;      /* [cap_rows] token row of each padded row, -1 for padding */
  int32_t* combine_plan; /* [T*k] receive-buffer row of token slot (t, j) in its owner's buffer, -1 if the
                            expert is not local */
  int32_t* scalars;      /* [5+R] M_pad, n_tiles, n_segs, N_r[0..R), n_mtiles, then the number of row tiles
                            that hold a row of another owner (they come first in mt_order) */
  int32_t* status;       /* [1] device status word (moe_status) */
  int32_t* mtile_desc;   /* [cap_mtiles][264] GEMM row tiles: {expert, n_rows, run_first, run_count,
                            self_lo, self_n, self_delta, 0, row[256]} (self_*: the expert's self-owned
                            group, first padded row, rows, receive row minus padded row), up to
                            256 (fp32: 64) real rows of one expert given by their
                            padded-layout positions, -1 past n_rows; each expert's groups are packed
                            together (self-owned group last) into the consecutive row tiles
                            [run_first, run_first + run_count) (internal schedule) */
  int32_t* seg_mtiles;   /* [cap_tiles][2] first GEMM row tile and count a segment depends on (internal) */
  int32_t* seg_sched;    /* [cap_tiles] segments in the order their row tiles complete (internal) */
  int32_t* chunk_counts; /* [R][ceil(T_o/64)][E_l] per-64-token histogram, then its prefix (internal) */
  int32_t* mt_order;     /* [cap_mtiles] the producer's row-tile order (remote first): every GEMM row tile that holds
                            a row of another owner, by number, then every row tile of self-owned rows only, by
                            number (internal schedule) */
  int64_t cap_rows;      /* capacity in padded rows (x_pad, h, y_pad, row_src) */
  int64_t cap_tiles;     /* cap_rows / M */
  int64_t cap_mtiles;    /* capacity of mtile_desc */
} moe_layout;

/* Knobs of moe_expert_ffn_overlap. */
typedef struct {
  int32_t consumer_cus;    /* C: consumer workgroups, one per CU, in [1, CUs/2]; the producer's persistent
                              launch runs one workgroup on each other CU.  0 = the launch picks C (0 included)
                              from the batch's routing and observed rates (see moe_pick_consumer_cus); -1 (bf16,
                              mode 0) = none: every workgroup produces, and takes copy units once its items are
                              done, so the return runs at the launch's tail */
  int32_t mode;            /* 0 = overlapped (the C consumer workgroups and the producer workgroups in one
                                  launch, on disjoint CUs; a producer workgroup joins the return once its
                                  own items are done),
                              1 = sequential (producer on all CUs, then the return on all CUs),
                              2 = return only (the consumer alone, on consumer_cus workgroups, for flags
                                  already published with this epoch; a flag never published ends in the
                                  watchdog; it delivers the other owners' rows, not the self owner's),
                              3 = return on the DMA engines (bf16): the producer's item list as a few launches
                                  on every CU, cut at window boundaries; after each, the segments it completed
                                  are copied with hipMemcpyDeviceToDeviceNoCU on a copy streams of the library
                                  while the next launch computes.  Reads the layout's segment table back first
                                  (synchronises `stream`); consumer_cus is not used */
  uint32_t epoch;          /* flag value of this call: nonzero and different from what the flag array holds
                              (flags start zeroed; pass 1, 2, 3, ...) */
  int32_t band_window;     /* GEMM row tiles per window of the producer's item list (0 = library default, 4):
                              the items of a window share weight tiles, and a window's second-GEMM items
                              follow the next window's first-GEMM items */
  uint64_t watchdog_ticks; /* spin budget of every wait in the launch (consumer and producer), 100 MHz ticks
                              (0 = 2 s); on expiry the status word becomes MOE_ETIMEOUT and the waiting
                              workgroup exits */
  uint64_t* timestamps;    /* optional (device) [2 + 2*cap_tiles] u64, 100 MHz clock: [0] first producer
                              item start, [1] last flag publish, [2+2s] / [3+2s] first copy start / last copy
                              end of segment s over the workgroups that copy it (a self-owned segment,
                              never copied, keeps ~0 / 0); reset by the call; NULL to skip */
  int32_t tile_order;      /* the producer's row-tile order (bf16): 0 = remote first (moe_layout.mt_order: every row
                              tile holding another owner's row before every row tile of self-owned rows only; the
                              review page's "Core claim"), 1 = row-tile numbering (each expert's rows together,
                              its self-owned rows last) */
  const void* x_tokens;    /* optional (device) [T, d] bf16 token rows, modes 0 and 1: the launch lands x_pad's real
                              rows itself (x_pad[p] = x_tokens[row_src[p]]), row tile by row tile in the order its
                              first GEMM needs them, each row tile's first-GEMM items waiting for that tile's rows
                              (review page, "Where Pith is reading between the lines": the dispatch side of the same
                              tile signalling).  For a layout built with x == NULL; NULL: x_pad already holds them */
  float* gu_out;           /* optional (device) [cap_rows, 2f] fp32 (bf16 with f a multiple of 128, as the backward
                              needs; modes 0, 1 and 3): the first GEMM's pre-activations of every real row at its
                              padded row, g = x Wg^T in columns [0, f) and u = x Wu^T in [f, 2f), as the fp32
                              accumulators hold them, for a backward call that takes them (moe_bwd_args.gu) instead of
                              recomputing that GEMM; rows of no real row are not written.  NULL: not stored */
} moe_overlap_cfg;

/* Last host-side error message of the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library build identifier, e.g. "moe_overlap gfx950". */
const char* moe_version(void);

/* ---- routing (input of the path) ----------------------------------------------------------------
 * Per token: top-k of G logits, descending, equal logits to the lower expert id; weight of a chosen
 * expert = softmax over all G logits at that id, not renormalised over the k (the router output the
 * review page's ledger, axiom 3, takes as known before the return).
 * logits (device) fp32 [T, G]; topk_idx (device) int32 [T, k]; topk_w (device) fp32 [T, k]. */
int moe_route(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/* ---- layout -------------------------------------------------------------------------------------- */

/* Capacity bound of the padded row count: T*min(k, E_l) + E_l*R*(M-1), rounded up to M.
 * Returns -1 for an invalid shape. */
int64_t moe_layout_capacity_rows(const moe_shape* s);

/* Bytes of device workspace that moe_layout_bind carves (256-byte aligned arrays); -1 if invalid. */
int64_t moe_layout_workspace_bytes(const moe_shape* s);

/* Host-only: point the arrays of *L into `workspace` (device, >= moe_layout_workspace_bytes bytes,
 * 256-byte aligned).  No device work. */
int moe_layout_bind(const moe_shape* s, void* workspace, int64_t workspace_bytes, moe_layout* L);

/* Build the remote-owner-aligned layout (review page: "What carries the argument"; referee major comment
 * 1 restating Algorithm 1): histogram of (expert, owner) groups, prefix scans and metadata, stable
 * scatter (rows of a group ascend by token), and the gather of token rows into x_pad.
 * topk_idx (device) int32 [T, k]; x (device) [T, d] in s->dtype; x_pad (device) [cap_rows, d].
 * Padding rows of x_pad are not written.  x == NULL skips the gather (x_pad is then not used and may be NULL):
 * for a bf16 FFN call that lands the rows itself (moe_overlap_cfg.x_tokens).  Resets the status word to MOE_OK first; sets MOE_ECAPACITY if
 * the padded rows exceed L->cap_rows (then all outputs are left empty: M_pad = 0). */
int moe_layout_build(const moe_shape* s, const int32_t* topk_idx, const void* x, moe_layout* L, void* x_pad,
                     void* stream);

/* Syncs `stream` and returns the device status word. */
int moe_read_status(const moe_layout* L, void* stream);

/* ---- expert FFN + return ------------------------------------------------------------------------- */

/* Size, in 4-byte words, of the flag buffer moe_expert_ffn_overlap needs; -1 if the shape is invalid.  It
 * holds the readiness flags of the second GEMM's output tiles (what the consumer waits on), and for bf16 the
 * flags of the first GEMM's h tiles, an arrival counter per output tile of the second GEMM and the fp32 partial
 * sums of its k-splits (256 x 256 floats per output tile and split; f/d rounded gives the number of splits, up
 * to 8); then one 64-bit counter of the return's copy units; for bf16 the landing's input flag and unit count per
 * row tile and its unit counter (moe_overlap_cfg.x_tokens); last (bf16), the MOE_OBS_WORDS words of the consumer
 * partition record (see moe_pick_consumer_cus).  Zero the buffer once before the first call; afterwards it is
 * epoch-valued. */
int64_t moe_ffn_flags_count(const moe_shape* s);

/* The consumer partition (review page: "If this is right" reports the overlap collapsing with too few consumer
 * SMs; "Where Pith is reading between the lines" proposes sizing the partition at run time).  With
 * cfg->consumer_cus = 0, an overlapped bf16 launch picks it itself, on the device, from this batch's routing (rows
 * routed to the local experts, rows to return to other owners: the layout's per-owner counts) and from rates it
 * observed in earlier calls on the same flag buffer: the producers' flops per CU and the consumers' copied bytes per
 * CU, per 100 MHz tick.  The rule: 0 (no partition: every workgroup takes copy units once its own items are
 * done) when, with the first-GEMM items (n_mtiles times f / 128 of them, each 2 x 256 x 256 x d flops) filling their
 * last round over the n_cu workgroups only in part, the workgroups without one of that round copy 4 d bytes per
 * returned row (at 50000 bytes per tick over the chip, or their own copy rate if lower) within one first-GEMM item's
 * time; else the smallest multiple of 8 in [8, min(32, n_cu/4)] at which the consumers alone would return the rows
 * in half the time the other CUs take for 6 d f flops per routed row.
 * The choice of the last overlapped call is word MOE_OBS_WORDS - 4 counted from the end of the flag buffer.
 * moe_pick_consumer_cus_observed evaluates the rule for given rows, row tiles and rates (a rate <= 0 takes its
 * default: 450 bytes and 31250 flops per CU-tick, ~45 GB/s and ~0.8 PFLOP/s over 256 CUs); moe_pick_consumer_cus for
 * the defaults with R - 1 of every R rows returned, in full row tiles.  fp32: 8 (at most a quarter of the CUs).  Host
 * only; -1 for an invalid shape or arguments, or n_cu < 2. */
int32_t moe_pick_consumer_cus(const moe_shape* s, int32_t n_cu);
int32_t moe_pick_consumer_cus_observed(const moe_shape* s, int32_t n_cu, int64_t rows_routed, int64_t rows_returned,
                                       int32_t n_mtiles, float ffn_rate, float copy_rate);
#define MOE_OBS_WORDS 16

/* Expert SwiGLU FFN over the padded layout with the return of each finished row-band segment to its
 * owner (review page: "The pith", "Core claim", "What carries the argument").
 *   h = bf16(silu(x Wg^T) * (x Wu^T)),  y = h Wd^T, per row with the row's local expert;
 *   Wg = rows [0, f) and Wu = rows [f, 2f) of w_gate_up[e].
 * The producer is one persistent launch over all local experts (bf16): tiles of h, then k-splits of y tiles,
 * window by window in remote-first row-tile order; a tile other workgroups read is published with an
 * epoch-valued flag once its stores are complete and visible device-wide.  That publish is not a release-scope
 * atomic: the tile is written with device-scope stores, their completion is awaited (vmcnt 0) and ordered by a
 * workgroup-scope release fence, and the flag is a relaxed agent-scope atomic store; readers drop stale lines
 * with one agent-scope acquire at the start of the launch.  An agent-scope release writes back the XCD's whole
 * L2 (measured: 0.23 ms of a 1.3 ms launch for the Mixtral-like shard's ~1,760 tiles).  The return is cut into copy units
 * of up to 128 KB of a segment, handed out in the order the segments complete: a workgroup in the consumer
 * role takes the next unit, waits for the flags of its segment's row tiles, acquires, and copies the unit's
 * rows into recv[owner].  The self owner's rows need no transfer (review page: the producer schedules the
 * remote-bound tiles first and the consumer moves those): the second GEMM stores them straight into
 * recv[self_rank], and its segments have no copy units.
 *   mode 0 (overlapped): the consumer is the first consumer_cus workgroups of the producer launch, and every
 *     producer workgroup joins it once its own items are done;
 *   mode 1 (sequential): producer on every CU, then the return alone on every CU;
 *   mode 2: the consumer alone (return only; for tests of the wait);
 *   mode 3: the return on the DMA engines instead of consumer CUs (the FiCCO review page's DMA offload), gated per
 *     launch chunk by events (see moe_overlap_cfg.mode).
 * fp32 runs the two GEMMs as two launches (consumer inside the second).  Owner r receives, at row
 * recv_off_{e,r} + i, the FFN output of the i-th row of group (e, r); results are identical in every mode.
 * y_pad holds the other owners' rows only (scratch of the return).
 * x_pad (device) [cap_rows, d]; w_gate_up (device) [E_l, 2f, d]; w_down (device) [E_l, d, f];
 * h_ws (device) [cap_rows, f] workspace; y_pad (device) [cap_rows, d]; recv: host array of R device
 * pointers, recv[r] holds >= N_r rows of d; flags (device, 8-byte aligned) [moe_ffn_flags_count] 4-byte
 * words (zeroed before the first call); cfg: see moe_overlap_cfg.  Waits inside the launch are bounded by cfg->watchdog_ticks;
 * on expiry the status word becomes MOE_ETIMEOUT. */
int moe_expert_ffn_overlap(const moe_shape* s, const moe_layout* L, const void* x_pad, const void* w_gate_up,
                           const void* w_down, void* h_ws, void* y_pad, void* const* recv, uint32_t* flags,
                           const moe_overlap_cfg* cfg, void* stream);

/* For callers that cannot allocate device memory or pass a workspace of their own (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): moe_expert_ffn_overlap without the `flags`
 * workspace.  The flag buffer (tile flags, split arrival counters, split-K partial sums, the copy-unit counter)
 * lives in a file-scope device array of the library, at most 64 MiB, which every device the library runs on
 * holds until the process ends; the call allocates nothing and calls no allocating routine.  Each call first
 * clears the flags and counters of that array with a fill kernel on `stream` and then runs with epoch 1
 * (cfg->epoch is ignored), so calls need no epoch sequence of their own.  All calls on one device share the
 * array: calls that overlap on one device (different streams, or host threads) race and give wrong results;
 * order them.  Inputs, outputs and the other workspaces (h_ws, y_pad) are the caller's, as for
 * moe_expert_ffn_overlap, whose arguments and results this call has.  MOE_EINVAL when the shape's flag buffer
 * (moe_ffn_flags_count words) exceeds the 64 MiB maximum, or for mode 2 (it needs an earlier call's flags);
 * MOE_EHIP if the array's device address cannot be obtained. */
int moe_expert_ffn_overlap_noalloc(const moe_shape* s, const moe_layout* L, const void* x_pad, const void* w_gate_up,
                                   const void* w_down, void* h_ws, void* y_pad, void* const* recv,
                                   const moe_overlap_cfg* cfg, void* stream);

/* The work-item list of the bf16 FFN launch (host only, no device call; for inspection and tests): which
 * workgroup runs which item, in what order, for a launch on n_cu CUs with cfg's mode, consumer_cus, band_window and
 * tile_order (consumer_cus 0: the launch's rule with default rates, every row of the row tiles at positions before
 * n_remote_mtiles counted as returned).  The review page ("Core claim", "What carries the argument")
 * describes one persistent GEMM over all local experts whose remote-bound tiles are scheduled first; the list is
 * the kernel's own (a header both compile).  Inputs are the layout's row tiles as the device built them:
 * mt_hdr [n_mtiles][4] = the first four fields of each mtile_desc entry {expert, rows, run_first, run_count},
 * mt_order [n_mtiles] = moe_layout.mt_order, n_remote_mtiles = the layout scalar after n_mtiles.  Output: items [n][8] int32, list index i = {workgroup, sequence
 * number in that workgroup, kind (1 = GEMM1 tile, 2 = GEMM2 k-split), row tile, column tile, split, half (-1 or
 * 0/1 for a half-width item), target (GEMM2: items that complete the y tile)}.  *n_items receives the list length;
 * items == NULL with cap == 0 only queries it.  MOE_EINVAL for fp32 (two plain launches, no list), an invalid
 * shape or configuration, row-tile headers out of range, or cap below the length. */
int moe_ffn_schedule(const moe_shape* s, int32_t n_cu, const moe_overlap_cfg* cfg, int32_t n_mtiles,
                     int32_t n_remote_mtiles, const int32_t* mt_hdr, const int32_t* mt_order, int32_t* items,
                     int64_t cap, int64_t* n_items);

/* ---- combine ------------------------------------------------------------------------------------- */

/* Top-k weighted combine at the owners (review page ledger, axiom 3: the combine plan is known from the
 * router output).  out[r*T_o+t] = sum over slots j ascending with plan >= 0 of
 * topk_w[t, j] * recv[r][plan[t, j]], fp32 accumulation, rounded to the element type; tokens with no local
 * expert get zeros.  topk_w (device) fp32 [T, k]; recv: host array of R device pointers; out (device)
 * [T, d]. */
int moe_combine(const moe_shape* s, const moe_layout* L, const float* topk_w, void* const* recv, void* out,
                void* stream);

/* ---- kernel timing ------------------------------------------------------------------------------- */

/* ---- backward pass ------------------------------------------------------------------------------
 * The review page ("Where Pith is reading between the lines") notes that MoE training's backward pass has the
 * forward's GEMM-then-transfer structure, so the same tile signalling applies.  Given dOut = dL/d(out) of the
 * combined output, per routed row (token t, slot weight w, local expert e), with g = x Wg^T, u = x Wu^T, s =
 * silu(g), h = bf16(s u) as in the forward:
 *   dY = bf16(w dOut[t]) (fp32 product),  dH = dY Wd,  dU = bf16(dH s),  dG = bf16(dH u silu'(g)),
 *   dX = bf16((dG | dU) (Wg | Wu)),  dWd[e] = sum dY^T h,  dWgu[e] = sum (dG | dU)^T x (fp32 over e's rows);
 * the rows' dX are returned to their token owners (the overlapped transfer), and the combine's backward gives
 * dx[t] = bf16(sum of t's delivered dX rows) and the routing weights' gradient <dOut[t], y>.  bf16 only; f a
 * multiple of 128. */
typedef struct {
  const int32_t* topk_idx; /* (device) [T, k] the forward's routing */
  const float* topk_w;     /* (device) [T, k] */
  const void* x_pad;       /* (device) [cap_rows, d] the forward's input rows (gathered or landed) */
  const void* w_gate_up;   /* (device) [E_l, 2f, d] */
  const void* w_down;      /* (device) [E_l, d, f] */
  const void* d_out;       /* (device) [T, d] bf16 gradient of the combined output */
  void* dy_pad;            /* (device) [cap_rows, d] workspace: dY rows in the padded layout */
  float* dh_ws;            /* (device) [cap_rows, f] fp32 workspace: dH */
  void* h_ws;              /* (device) [cap_rows, f] workspace: h, recomputed */
  void* dgu_ws;            /* (device) [cap_rows, 2f] workspace: dG | dU */
  void* dx_pad;            /* (device) [cap_rows, d] workspace: dX rows of the other owners */
  void* const* dx_recv;    /* host array of R device pointers: owner r receives the dX of its rows at the rows where
                              the forward delivered their y (recv_off layout) */
  float* dw_gate_up;       /* (device) [E_l, 2f, d] fp32 weight gradient, written (not accumulated) */
  float* dw_down;          /* (device) [E_l, d, f] fp32 weight gradient, written */
  const float* gu;         /* optional (device) [cap_rows, 2f] fp32: g | u as the forward call of this layout and these
                              weights stored them (moe_overlap_cfg.gu_out); the h / dG / dU items then read them
                              instead of recomputing the first GEMM, with the same bits (the forward's first GEMM
                              and the recompute run the same k-tiles in the same order).  NULL: recompute */
} moe_bwd_args;

/* Size, in 4-byte words, of the backward call's flag buffer (dX tile flags first, then dH and h flags, the k-split
 * arrival counters and fp32 partial sums of dX, the copy-unit counter); -1 for an invalid shape, fp32, or f not a
 * multiple of 128.  Zero it once; afterwards it is epoch-valued like the forward's. */
int64_t moe_bwd_flags_count(const moe_shape* s);

/* The backward of the expert FFN with the return of the rows' dX to their owners: the dY rows (k_bwd_dy), then one
 * persistent launch of tile items (dH, then h / dG / dU, then dX with the split-K partial sums summed in split
 * order, then the weight gradients), each publishing an epoch-valued flag that later items and the consumer role
 * wait on; the consumer copies each finished segment's dX rows into dx_recv[owner] (the self owner's rows are
 * stored there by the dX items).  cfg: mode 0 = overlapped (every workgroup runs its share of the dH, h / dG / dU
 * and dX items; then the first consumer_cus workgroups return rows while the others take weight-gradient tiles, and
 * join those once every copy unit is handed out; every workgroup takes the copy units left at the end; 0 and -1 =
 * none: the return after the weight-gradient tiles, on every workgroup, which on one device is the faster), mode 1 =
 * sequential (the producers, then the return on every CU); epoch and watchdog_ticks as in the forward; results
 * are identical in both modes.  The layout must be the forward's (moe_layout_build of the same routing). */
int moe_expert_ffn_backward(const moe_shape* s, const moe_layout* L, const moe_bwd_args* b, uint32_t* flags,
                            const moe_overlap_cfg* cfg, void* stream);

/* The combine's backward: dx (device, bf16 [T, d]) = per token the fp32 sum, in slot order, of its delivered dX rows
 * (dx_recv, as moe_expert_ffn_backward fills them), rounded once; dw_route (device, fp32 [T, k]) = <dOut[t], y_j>
 * over the forward's delivered rows y_recv (0 for slots routed elsewhere).  Tokens with no local slot get zero
 * rows.  bf16 only. */
int moe_combine_backward(const moe_shape* s, const moe_layout* L, const void* d_out, void* const* y_recv,
                         void* const* dx_recv, void* dx, float* dw_route, void* stream);

/* While enabled (nonzero), every moe_expert_ffn_overlap and moe_expert_ffn_backward call of this process times
 * each of its launches with a pair of HIP events that the launch itself records (hipExtLaunchKernel: the kernel's start and end, no marker
 * in the caller's stream).  Disabled by default.  Returns MOE_OK. */
int moe_set_kernel_timing(int enable);

/* Waits for the recorded events and writes the summed milliseconds since the last query:
 * out[0] the producer launch (bf16: the whole FFN, with the consumer workgroups in overlapped mode; fp32: the
 * first GEMM), out[1] the second launch (fp32: the second GEMM with the consumer workgroups; bf16: 0),
 * out[2] the separate consumer launch of sequential mode (0 in overlapped mode), out[3] number of calls
 * recorded.  Clears the record. */
int moe_kernel_times(double* out4);

#ifdef __cplusplus
}
#endif

#endif /* MOE_OVERLAP_H */
