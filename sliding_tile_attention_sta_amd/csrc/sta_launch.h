// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sta {

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  const int32_t *sched;    // work items in launch order (-1 = idle)
  const int32_t *kv_off;   // heads*n_tiles + 1
  const int32_t *kv_idx;   // key tiles of each (head, query tile)
  const int32_t *base;     // n_tiles: first token row of each tile in the tensors' layout
  const int32_t *off;      // tile_tokens: row offset of each tile-local token
  int32_t heads, n_tiles, V, subs;
  int64_t N;               // tokens per (batch, head)
  float sl2e;              // softmax scale * log2(e)
  int32_t n_blocks;        // length of sched
  int32_t max_nkv;         // longest key-tile list of any (head, query tile)
  float *lse;              // NULL, or [batch, heads, N] row log-sum-exp (natural log)
  int32_t sep;             // rows of a 32-key block = its first row + a per-position offset
                           // (and the step table fits in LDS): per-step addressing
  const uint32_t *kmask;   // NULL (whole tiles), or per tile V/32 words of token validity
  // Token-wise SWA plans only (swin == NULL otherwise): clamped token
  // windows per head (heads*3), extents, query tile sizes, query tile grid.
  const int32_t *swin;
  int32_t T, H, W, tT, tH, tW, gH, gW;
  // Dynamic queues (NULL: work group b runs sched[b]): the 8 XCD queues and
  // the piece queue concatenated, queue k at queue[qoff[k] .. qoff[k+1]),
  // and the launch's queue words (scratch; zero between launches).
  const int32_t *queue;
  int32_t qoff[10];
  int32_t *qcount;         // scratch queue words (also the fix-up count and done counter)
  // Work items whose O came out non-finite (V beyond fp16's range): a bit
  // per item code and the list of marked items (scratch; zero between
  // launches).
  unsigned *fbits;
  int32_t *flist;
  // Work items split by key range (entries -2 - p): per piece (item, first
  // step, end step, group), per group (first piece, pieces), and the
  // launch's scratch: an arrival counter per group (zero between launches)
  // and a partial-result slot per piece.  NULL when there are no pieces.
  const int32_t *ptab;
  const int32_t *gtab;
  int32_t *pcount;
  float *pslot;
  // Per-work-group lists (NULL otherwise): work group b runs the codes
  // wlist[woff[b] .. woff[b+1]) in turn (whole items and pieces).
  const int32_t *wlist;
  const int32_t *woff;
  int32_t n_items, n_pieces;   // item codes in [0, n_items), pieces in [0, n_pieces)
  unsigned *dbg;               // debug builds: bounds-check violation bits (else unused)
};

// Zero n int32 (a fill kernel, so that the clear can sit in a captured graph).
hipError_t launch_zero(int32_t *p, int n, hipStream_t stream);

// Launch the forward kernel.  variant: 0 generic, 1 384-query items.
hipError_t launch_forward(const FwdArgs &a, int variant, int head_dim, bool f32_in, bool f32_out,
                          hipStream_t stream);

struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *lse;        // [batch, heads, N], natural log
  const float *delta;      // [batch, heads, N], rowsum(dO * O)
  void *dq, *dk, *dv;
  const int32_t *sched;    // work items in launch order (-1 = idle)
  const int32_t *list_off; // dQ: key-tile lists per (head, query tile); dK/dV: query-tile lists
  const int32_t *list_idx;
  const int32_t *base;     // n_tiles: first token row of each tile in the tensors' layout
  const int32_t *off;      // tile_tokens: row offset of each tile-local token
  const uint32_t *kmask;   // partial plans: n_tiles * V/32 token validity words (else null)
  int32_t heads, n_tiles, V, subs;
  int64_t N;
  float scale;             // softmax scale
  float sl2e;              // scale * log2(e)
  int32_t n_blocks;        // length of sched
  int32_t max_list;        // longest list
  int32_t f32_out;         // gradients stored as fp32 (else bf16)
  int32_t n_items;         // work item codes in [0, n_items)
  unsigned *dbg;           // debug builds: bounds-check violation bits (else unused)
};

// delta[r] = sum_d dO[r, d] * O[r, d] for rows r < rows.
hipError_t launch_bwd_delta(const void *o, const void *dout, float *delta, int64_t rows, int head_dim,
                            bool f32_o, bool f32_g, hipStream_t stream);
// dQ kernel with nw waves of 32 queries per work item; dK/dV kernel with
// `pairs` wave pairs of 32 keys per work item.
hipError_t launch_bwd_dq(const BwdArgs &a, int nw, int head_dim, bool f32_in, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs &a, int pairs, int head_dim, bool f32_in, hipStream_t stream);

struct ReorderArgs {
  const void *in;
  void *out;
  const int32_t *base;     // natural-order base row of each tile
  const int32_t *off;      // natural-order offset of each tile-local token
  int64_t rows;            // batch*heads*N
  int64_t N;
  int32_t V;
  int32_t row_bytes;       // head_dim * element size, a multiple of 16
  int32_t inverse;         // 0: natural -> tile-major, 1: tile-major -> natural
};

hipError_t launch_reorder(const ReorderArgs &a, hipStream_t stream);

}  // namespace sta
