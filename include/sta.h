/*
 * sta.h -- C ABI of the MI355X (gfx950) Sliding Tile Attention library (forward and backward).
 *
 * Operation (source: "Fast Video Generation with Sliding Tile Attention",
 * arXiv 2502.04507 -- index page, section "Abstract"; gptget summary page,
 * sections "Methodology", "Technical Contribution" and "Novelty"):
 * a T x H x W video latent is cut into non-overlapping tiles of
 * tT x tH x tW tokens; every query tile attends to all tokens of exactly the
 * key/value tiles inside its 3D window (a box of wT x wH x wW tiles, chosen
 * per head), and to nothing else, so no (query tile, key tile) block is ever
 * partly masked.  Inside the window it is ordinary softmax attention:
 *
 *     O[x] = sum_j softmax_j(scale * Q[x].K[j]) V[j],  j over the window.
 *
 * Window geometry: a window wider than the tile grid is clamped to it; the
 * window of query tile c on an axis of n tiles starts at
 * clamp(c - floor((w-1)/2), 0, n - w), so border windows shift inward and
 * every query tile sees exactly wT*wH*wW key tiles.
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned DEVICE pointers, contiguous
 *     [batch, heads, N, head_dim] with N = T*H*W tokens.  In
 *     STA_LAYOUT_NATURAL the token axis is raster order (t, y, z), z fastest,
 *     i.e. the tensor is [batch, heads, T, H, W, head_dim].  In
 *     STA_LAYOUT_TILE_MAJOR each tile's tokens are contiguous: tiles in
 *     raster order of tile coordinates, tokens inside a tile in raster order
 *     of their local (t, y, z).
 *   - out must not overlap any input.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous with respect to the host; none synchronises.
 *   - Every argument and shape check runs on the host before any launch, so a
 *     call that returns an error has written nothing.
 *   - Functions never throw; they return a sta_status.
 *   - A plan is immutable after creation; it may be used from several host
 *     threads and streams at once.  Its device tables are uploaded once per
 *     device, on the first call that needs them.
 *   - Test hook: with STA_TEST_FAIL_ALLOC=1 in the environment (read at
 *     every allocation), every plan, device-table and scratch allocation of
 *     the library fails and the call returns STA_ERR_ALLOC, leaking nothing.
 */
#ifndef STA_H
#define STA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STA_OK = 0,
  STA_ERR_ARG = -1,         /* null pointer, window < 1, bad enum, scale <= 0, ... */
  STA_ERR_SHAPE = -2,       /* an extent is not a positive multiple of its tile size */
  STA_ERR_UNSUPPORTED = -3, /* head_dim not 64/128, or tile volume not a multiple of 32 */
  STA_ERR_ALLOC = -4,       /* host or device allocation failed */
  STA_ERR_HIP = -5          /* a HIP runtime call or a launch failed (incl. no device) */
} sta_status;

typedef enum { STA_BF16 = 0, STA_F32 = 1 } sta_dtype;

typedef enum { STA_LAYOUT_NATURAL = 0, STA_LAYOUT_TILE_MAJOR = 1 } sta_layout;

/* Flags of sta_plan_create_ex. */
enum { STA_PLAN_PARTIAL_TILES = 1 };

typedef struct sta_plan sta_plan; /* opaque, owned by the library */

/* Read-only description of a plan (host memory, filled by sta_plan_get_info). */
typedef struct {
  int32_t batch, heads, T, H, W, head_dim;
  int32_t tile[3];          /* tokens per tile on (T, H, W) */
  int32_t grid[3];          /* tiles on (T, H, W) */
  int32_t tile_tokens;      /* tT*tH*tW */
  int32_t n_tiles;          /* grid[0]*grid[1]*grid[2] */
  int64_t tokens;           /* T*H*W */
  int64_t pairs;            /* attended (query tile, key tile) pairs, summed over heads, one batch element */
  double flops;             /* 4 * tile_tokens^2 * head_dim * pairs * batch: FLOPs of the two products */
  int64_t work_items;       /* entries of the forward schedule (sta_plan_schedule): work items,
                               idle padding and pieces */
  int32_t queries_per_item; /* query tokens per work item */
  int32_t kernel_variant;   /* 0 = generic (32 queries / item), 1 = 384-query items */
  int32_t bwd_supported;    /* 1 if sta_backward_plan accepts this plan */
  int32_t bwd_queries_per_item; /* queries per dQ work item */
  int32_t bwd_keys_per_item;    /* keys per dK/dV work item */
  int64_t bwd_items_dq;     /* launched dQ work items (including idle padding) */
  int64_t bwd_items_dkdv;   /* launched dK/dV work items (including idle padding) */
  int32_t partial_tiles;    /* 1 if some extent is not a multiple of its tile size */
  int32_t swa;              /* 1 for a token-wise sliding-window plan (sta_swa_plan_create) */
  int32_t split_items;      /* forward work items split by key range (0 = none) */
  int32_t pieces;           /* launched pieces of those items */
  int64_t scratch_bytes;    /* device scratch a forward launch of this plan uses (queue and
                               arrival counters, fix-up marks, partial results of pieces) */
  int64_t launch_blocks;    /* work groups of one forward launch (256 with per-work-group
                               lists, see sta_plan_group_lists) */
} sta_plan_info;

/* Source: "Fast Video Generation with Sliding Tile Attention", index page,
 * Abstract (non-overlapping 3D tiles, a window of whole tiles per query
 * tile, window size set per head); gptget summary page, Methodology (the
 * window slides tile by tile, so every (query tile, key tile) block is
 * either fully attended or skipped).
 * Build the host plan: tile grid, clamped per-head windows, per-(head, query
 * tile) key-tile lists (raster order of tile coordinates) and the launch
 * schedule (work items ordered by decreasing cost, spread evenly over the
 * chip's XCDs).  Host work only; no device is touched.
 *   window: heads*3 ints (wT, wH, wW) in tiles, >= 1; wider than the grid is clamped.
 *   tile:   3 ints (tT, tH, tW) in tokens.
 * Errors: STA_ERR_ARG (null, non-positive sizes or windows), STA_ERR_SHAPE
 * (T, H or W not a multiple of its tile size), STA_ERR_UNSUPPORTED (head_dim
 * not 64 or 128; tile volume not a multiple of 32 or above 4096;
 * batch*heads*T*H*W above INT32_MAX; more than INT32_MAX (head, query tile,
 * key tile) pairs; a key-tile list too long for the forward kernel's LDS),
 * STA_ERR_ALLOC.
 * On success *out owns the plan; release it with sta_plan_destroy. */
sta_status sta_plan_create(int batch, int heads, int T, int H, int W, const int tile[3],
                           const int *window, int head_dim, sta_plan **out);

/* As sta_plan_create, with flags.  STA_PLAN_PARTIAL_TILES accepts extents
 * that are not multiples of their tile size (the pages leave such latents
 * open; reading used: an axis then has ceil(extent / tile) tiles, its last
 * tile partial, windows and tile geometry unchanged, and only tokens that
 * exist take part -- the same as padding the video to whole tiles and
 * masking the padded keys).  Such a plan supports sta_forward_plan,
 * sta_forward_plan_lse and sta_backward_plan in STA_LAYOUT_NATURAL only
 * (the gradients of tokens that do not exist are not defined and nothing
 * is written for them); sta_plan_perm, sta_tile_reorder/unreorder and the
 * tile-major layout return STA_ERR_UNSUPPORTED for it.  Its info.flops
 * counts whole tiles (the work performed).  STA_ERR_ARG for unknown flags. */
sta_status sta_plan_create_ex(int batch, int heads, int T, int H, int W, const int tile[3],
                              const int *window, int head_dim, int flags, sta_plan **out);

/* Token-wise 3D sliding window attention, the baseline the pages contrast
 * STA with (index page, Abstract; gptget summary page, Methodology and
 * Novelty): every query token attends to the keys of its own window of
 * window_tokens[3h .. 3h+2] tokens (per head; clamped to the extents),
 * centred on it and shifted inward at the borders (the same rule as STA's
 * window, at token level).  The plan groups queries into work items of
 * tile[3] tokens (extents must be multiples of it); a work item walks the
 * union of its queries' windows in runs of 32 keys and masks every score
 * against its query's window, so its blocks are "mixed".  Run it with
 * sta_forward_plan / sta_forward_plan_lse in STA_LAYOUT_NATURAL;
 * info.flops counts the permitted (query, key) pairs only.  Tile-major
 * layout, reorder, perm and backward return STA_ERR_UNSUPPORTED.
 * Errors: as sta_plan_create. */
sta_status sta_swa_plan_create(int batch, int heads, int T, int H, int W, const int tile[3],
                               const int *window_tokens, int head_dim, sta_plan **out);

/* Release a plan and its device tables (NULL is a no-op).  Before freeing
 * the tables on a device it waits for all work queued on that device
 * (hipDeviceSynchronize), so a plan may be released right after launching
 * work with it; it must not be released while another host thread is still
 * launching with it. */
sta_status sta_plan_destroy(sta_plan *plan);

/* Copy the plan description into *info (host). */
sta_status sta_plan_get_info(const sta_plan *plan, sta_plan_info *info);

/* Tile-major position -> natural token index, for all N tokens.
 * perm: host buffer of at least cap int32.  STA_ERR_ARG if cap < N. */
sta_status sta_plan_perm(const sta_plan *plan, int32_t *perm, int64_t cap);

/* Key tiles (raster tile indices, ascending) of query tile q_tile for head
 * head.  out: host buffer of cap int32; *count receives the list length even
 * when it exceeds cap (then STA_ERR_ARG and out holds the first cap entries). */
sta_status sta_plan_kv_tiles(const sta_plan *plan, int head, int q_tile, int32_t *out, int cap,
                             int *count);

/* The same lists in the order the kernels walk them.  which = 0: the key
 * tiles of query tile `tile` as the forward (and the backward's dQ kernel)
 * visit them: raster order of (a mod wT, b mod wH, c mod wW) over the
 * tile's window, a one-to-one map on any w consecutive tiles per axis, so
 * query tiles whose windows overlap reach their shared key tiles at the
 * same step.  which = 1: the query tiles whose window holds key tile
 * `tile`, as the dK/dV kernel visits them: by the same residue of the query
 * tile's coordinates, ties in raster order.  Buffer and error conventions
 * as sta_plan_kv_tiles; STA_ERR_ARG also for token-wise SWA plans (no
 * lists). */
sta_status sta_plan_walk(const sta_plan *plan, int which, int head, int tile, int32_t *out, int cap,
                         int *count);

/* Query tiles (raster indices, ascending) whose window holds key tile
 * kv_tile for head head: the inverse of sta_plan_kv_tiles, walked by the
 * backward's dK/dV kernel.  Buffer and error conventions as sta_plan_kv_tiles. */
sta_status sta_plan_q_tiles(const sta_plan *plan, int head, int kv_tile, int32_t *out, int cap,
                            int *count);

/* The forward's work queues, one per XCD (accelerator complex die) of the
 * chip, interleaved: entry s * 8 + x is the s-th entry of XCD x's queue,
 * -1 where that queue is shorter than the longest.  Other entries are item
 * codes, or -2 - p for piece p of a split item (see sta_plan_pieces).  A
 * code >= 0 encodes ((b * heads + h) * n_tiles + q_tile) * subs + sub,
 * where subs = tile_tokens / queries_per_item.  With the 384-query kernel
 * (info.kernel_variant 1) the queues are consumed dynamically: each work
 * group takes the next entry of its own XCD's queue, or, once that queue
 * is empty, of another's, so a faster XCD takes more of the work; otherwise
 * work group b runs entry b.  Plans of the 384-query kernel with fewer
 * work items than the chip's 256 compute units may instead cut the
 * launch's key steps into one contiguous range per work group (see
 * sta_plan_group_lists): the schedule is then the groups' lists,
 * concatenated.  out: host buffer of cap int32; *count receives the entry
 * count (STA_ERR_ARG if it exceeds cap). */
sta_status sta_plan_schedule(const sta_plan *plan, int32_t *out, int64_t cap, int64_t *count);

/* Per-work-group lists of the forward (plans with fewer work items than
 * compute units, where balancing the units' key steps pays): work group b
 * runs the schedule's entries off[b] .. off[b + 1] - 1 in turn, whole items
 * and pieces (see sta_plan_pieces) that together walk one contiguous range
 * of the launch's key steps, the items taken in decreasing-cost order.
 * out: host buffer of cap int32 that receives info.launch_blocks + 1
 * offsets; *count receives that number, or 0 when the plan has no such
 * lists (STA_ERR_ARG if it exceeds cap). */
sta_status sta_plan_group_lists(const sta_plan *plan, int32_t *out, int64_t cap, int64_t *count);

/* The pieces of split work items (info.pieces of them).  A work item of the
 * forward walks its key tiles' 32-key blocks in order, steps
 * 0 .. key_tiles * tile_tokens / 32 - 1; when equal-cost items would leave
 * the last round of a launch to a few compute units, the plan cuts those
 * items into pieces of consecutive steps that run side by side, and the
 * last piece of an item to finish combines the pieces' partial softmax
 * results (exact up to fp32 rounding: each piece's unnormalised output and
 * row sums are rescaled to the largest of their reference maxima).
 * out: host buffer of cap * 5 int32, per piece (item code, first step, end
 * step, item index among the split items, pieces of that item); *count
 * receives the piece count (STA_ERR_ARG if it exceeds cap). */
sta_status sta_plan_pieces(const sta_plan *plan, int32_t *out, int64_t cap, int64_t *count);

/* The backward schedules, same conventions: which = 0 for the dQ kernel
 * (code ((b * heads + h) * n_tiles + q_tile) * subs + sub, subs =
 * tile_tokens / bwd_queries_per_item), 1 for the dK/dV kernel (the same
 * with the key tile and bwd_keys_per_item).  Empty when bwd_supported is 0. */
sta_status sta_plan_schedule_bwd(const sta_plan *plan, int which, int32_t *out, int64_t cap,
                                 int64_t *count);

/* Source: "Fast Video Generation with Sliding Tile Attention", gptget
 * summary page, Technical Contribution (a tile-based design aligned with the
 * hardware, which minimizes irregular memory access).  Reading used: the
 * tokens of each tile are made contiguous in memory (tile-major order), so
 * that every (query tile, key tile) pair is one dense block; the inverse
 * permutation restores the video's raster order.
 * Gather a [batch, heads, N, head_dim] tensor from natural into tile-major
 * token order (out[.., p, :] = in[.., perm[p], :]), or back.  dtype is the
 * element type of both tensors.  Bound by HBM bandwidth. */
sta_status sta_tile_reorder(const sta_plan *plan, const void *in, void *out, sta_dtype dtype,
                            void *stream);
sta_status sta_tile_unreorder(const sta_plan *plan, const void *in, void *out, sta_dtype dtype,
                              void *stream);

/* Source: "Fast Video Generation with Sliding Tile Attention", index page,
 * Abstract, and gptget summary page, Methodology: inside its window a query
 * tile takes ordinary softmax attention over every key of the window's
 * tiles (the formula at the top of this file); no block is partly masked.
 * STA forward with a plan.  q, k, v: [batch, heads, N, head_dim] of in_dtype;
 * out: same shape, out_dtype (STA_F32 or STA_BF16).  All four tensors use the
 * token order given by layout.  scale > 0 multiplies Q.K (usually
 * 1/sqrt(head_dim)).
 * Precision: Q.K^T runs on bf16 MFMA (STA_F32 q and k are rounded to bf16,
 * nearest-even, as they are loaded); the softmax runs in fp32; P.V runs on
 * fp16 MFMA with P rounded to fp16 and V converted to fp16 (exact for bf16
 * values, nearest-even for fp32), all accumulated in fp32.  V beyond the
 * fp16 range (|v| > 65504, possible in bf16 and fp32): a work item whose
 * output comes out non-finite is redone by a second kernel of the same
 * call with V multiplied by 2^-e and O by 2^e (e from the largest |v| of
 * the item's keys), so any finite V gives a finite, correctly scaled O.
 * Inputs must be finite.  The result does not depend on the order in which
 * key tiles are visited beyond fp32 rounding. */
sta_status sta_forward_plan(const sta_plan *plan, const void *q, const void *k, const void *v,
                            void *out, float scale, sta_dtype in_dtype, sta_dtype out_dtype,
                            sta_layout layout, void *stream);

/* STA forward that also writes the row log-sum-exp the backward needs.
 *   lse: caller-owned device buffer of batch*heads*N float, same token order
 *        as layout; lse[x] = ln(sum_j exp(scale * q_x.k_j)) over the keys of
 *        x's window (natural log, scale applied), computed from the same
 *        rounded probabilities as out.
 * Everything else as sta_forward_plan; lse must not overlap any tensor.
 * STA_ERR_ARG for a NULL lse. */
sta_status sta_forward_plan_lse(const sta_plan *plan, const void *q, const void *k, const void *v,
                                void *out, float *lse, float scale, sta_dtype in_dtype,
                                sta_dtype out_dtype, sta_layout layout, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as sta_forward_plan / sta_forward_plan_lse (lse may be NULL), with
 * no hipMalloc, hipFree or other allocating call.  Its work queues, arrival
 * counters and partial results use a fixed scratch array of 64 MiB that
 * each device holds while the library is loaded; the call clears the
 * counters with a small kernel on stream before the forward kernel.  Every
 * call on one device shares that device's array, so calls that overlap on
 * one device (different streams, host threads) race: serialise them.
 * The plan's tables must already be on the current device (any earlier
 * allocating call with the plan there -- sta_forward_plan, _lse,
 * sta_backward_plan, sta_tile_reorder -- uploads them).
 * Errors: as sta_forward_plan; STA_ERR_UNSUPPORTED if the plan's tables are
 * not on the device yet or its scratch (sta_plan_info.scratch_bytes) is
 * larger than 64 MiB. */
sta_status sta_forward_plan_noalloc(const sta_plan *plan, const void *q, const void *k, const void *v,
                                    void *out, float *lse, float scale, sta_dtype in_dtype,
                                    sta_dtype out_dtype, sta_layout layout, void *stream);

/* STA backward: gradients of <out, dout> with respect to q, k and v, where
 * out is STA's output for (q, k, v).  Defined by the chain rule of the
 * forward (the pages fine-tune through the operator; index page, Abstract,
 * and gptget summary page, Summary): with P_xj = exp(scale q_x.k_j - lse_x)
 * over the keys j of x's window,
 *     dv_j = sum_x P_xj dout_x
 *     dS_xj = P_xj (dout_x.v_j - delta_x),  delta_x = dout_x . out_x
 *     dq_x = scale sum_j dS_xj k_j,        dk_j = scale sum_x dS_xj q_x
 * where x runs over the queries whose window holds key j.
 *   q, k, v, dout: [batch, heads, N, head_dim] of in_dtype.
 *   out: the forward's output, out_dtype; lse: the forward's row log-sum-exp
 *        (sta_forward_plan_lse with the same q, k, v, scale and plan).
 *   delta: caller-owned device scratch of batch*heads*N float, overwritten
 *        with delta_x.
 *   dq, dk, dv: outputs, grad_dtype (STA_F32 or STA_BF16), same shape.
 * All tensors use the token order given by layout.  Written buffers (delta,
 * dq, dk, dv) must not overlap each other or any input.
 * Precision: every product runs on fp16 MFMA with fp32 accumulation; q and k
 * enter as the bf16 values the forward used (STA_F32 inputs rounded to bf16,
 * nearest-even), v and dout are converted to fp16 (exact for bf16 values in
 * range, nearest-even for fp32), and P and dS are rounded to fp16.  Entries
 * of q, k, v and dout and the products dS must lie within the fp16 range.
 * Deterministic: no atomics; dq and dk/dv come from separate kernels.
 * Partial-tile plans (sta_plan_create_ex): natural layout only; only
 * existing tokens take part, as in the forward.
 * Errors: STA_ERR_ARG (NULL, bad enum, scale <= 0, overlap),
 * STA_ERR_UNSUPPORTED (the plan's tile volume and window lists exceed the
 * backward kernels' LDS; a partial-tile plan in the tile-major layout),
 * STA_ERR_HIP. */
sta_status sta_backward_plan(const sta_plan *plan, const void *q, const void *k, const void *v,
                             const void *out, const void *dout, const float *lse, float *delta,
                             void *dq, void *dk, void *dv, float scale, sta_dtype in_dtype,
                             sta_dtype out_dtype, sta_dtype grad_dtype, sta_layout layout,
                             void *stream);

/* Same, building (or finding in a process-wide cache keyed by every shape
 * and window argument) the plan itself; extents that are not multiples of
 * the tile get a plan with partial tiles (as STA_PLAN_PARTIAL_TILES of
 * sta_plan_create_ex: natural layout only).  Cached plans live until
 * sta_clear_plan_cache or process exit.  Thread-safe: several threads may
 * call it at once, also while another clears the cache. */
sta_status sta_forward(const void *q, const void *k, const void *v, void *out, int batch, int heads,
                       int T, int H, int W, const int tile[3], const int *window, int head_dim,
                       float scale, sta_dtype in_dtype, sta_dtype out_dtype, sta_layout layout,
                       void *stream);

/* ---- Per-head window search -------------------------------------------
 * The pages configure each head's window automatically from the profiled
 * locality of its attention (index page, Abstract; gptget summary page,
 * Methodology, Technical Contribution and Limitations), giving no formula.
 * Reading implemented here: on calibration inputs, the error of candidate
 * window c for head h is ||O_c - O_full|| / ||O_full|| (Frobenius norm over
 * the batch, tokens and channels of head h, O_full = attention over the
 * whole video); each head gets the cheapest candidate, cost =
 * prod(min(w, grid)) key tiles per query tile, whose error is at most a
 * threshold (ties: smaller error, then earlier candidate), else the full
 * window (the grid). */

/* err[h * n_cand + c] for the candidate windows candidates[3c .. 3c+2] (in
 * tiles) on one calibration input q, k, v ([batch, heads, N, head_dim] of
 * in_dtype, DEVICE pointers, token order of layout).  err: HOST buffer of
 * heads * n_cand doubles.  Runs the forward once with the full window and
 * once per candidate (all heads at once) on stream, with fp32 outputs; the
 * library allocates two fp32 [batch, heads, N, head_dim] device buffers for
 * the call and frees them, and the call synchronises stream.  Extents that
 * are not multiples of the tile use plans with partial tiles
 * (STA_PLAN_PARTIAL_TILES of sta_plan_create_ex; grid = ceil(extent /
 * tile), natural layout only: STA_ERR_UNSUPPORTED for the tile-major one).
 * Errors: as sta_plan_create_ex and sta_forward_plan; STA_ERR_ALLOC. */
sta_status sta_window_errors(const void *q, const void *k, const void *v, int batch, int heads, int T,
                             int H, int W, const int tile[3], int head_dim, float scale,
                             sta_dtype in_dtype, sta_layout layout, const int *candidates,
                             int n_cand, double *err, void *stream);

/* Host only.  window_out[3h .. 3h+2] = the window chosen for head h from
 * err (heads x n_cand, e.g. sta_window_errors averaged over several
 * calibration inputs) under threshold, by the rule above.  grid: tiles on
 * (T, H, W).  STA_ERR_ARG on NULL or non-positive sizes. */
sta_status sta_window_select(int heads, const int grid[3], const int *candidates, int n_cand,
                             const double *err, double threshold, int *window_out);

/* The whole search over n_samples calibration inputs: q[s], k[s], v[s]
 * (arrays of n_samples DEVICE pointers, each tensor as in
 * sta_window_errors).  For every sample, the errors of sta_window_errors;
 * their arithmetic mean over the samples, summed in sample order (the
 * pages' per-head configuration reads several prompts; reading: errors
 * averaged before the choice); window_out[3h .. 3h+2] = the window that
 * sta_window_select chooses from the mean under threshold.  err_out: HOST
 * buffer of heads * n_cand doubles for the mean errors, or NULL.  The call
 * synchronises stream.
 * Errors: as sta_window_errors; STA_ERR_ARG for n_samples < 1 or a NULL
 * pointer in the arrays. */
sta_status sta_window_search(const void *const *q, const void *const *k, const void *const *v,
                             int n_samples, int batch, int heads, int T, int H, int W, const int tile[3],
                             int head_dim, float scale, sta_dtype in_dtype, sta_layout layout,
                             const int *candidates, int n_cand, double threshold, double *err_out,
                             int *window_out, void *stream);

/* Host only.  The default candidate set for a grid: on each axis every odd
 * extent below the axis length, and the axis length itself; all
 * combinations in raster order, written as triples to out (cap triples).
 * *count receives the number of candidates even when it exceeds cap (then
 * STA_ERR_ARG). */
sta_status sta_window_candidates(const int grid[3], int *out, int cap, int *count);

/* Drop every cached plan.  Safe while other threads are in sta_forward: a
 * plan that a call is still using is destroyed when that call returns. */
sta_status sta_clear_plan_cache(void);

/* Debug builds only (libsta_debug.so, compiled with -DSTA_DEBUG): the
 * kernels check work item codes, tile-list entries, token rows, buffer
 * offsets and LDS table indices, and a failed check sets a bit in a word on
 * the current device instead of trapping (bits: 0 work item or piece,
 * 1 tile-list entry, 2 row or offset of a load, 3 row of a store, 4 LDS
 * table index).  *flags receives the word (after the work queued before the
 * call on the null stream has finished); clear != 0 resets it.  Release
 * builds: *flags = 0 and STA_ERR_UNSUPPORTED.  STA_ERR_ARG for a NULL
 * flags, STA_ERR_HIP if the device cannot be read. */
sta_status sta_debug_flags(uint32_t *flags, int clear);

/* Static, human-readable name of a status code. */
const char *sta_status_string(sta_status status);

#ifdef __cplusplus
}
#endif

#endif /* STA_H */
