// Internal definitions shared by the host plan (sta_plan.cpp) and the HIP
// entry points (sta_api.hip).  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "sta.h"

namespace sta {

// Kernel variants: how many query tokens one work group owns.
enum Variant : int32_t {
  kGeneric = 0,   // 32 queries per work item (2 waves x 16); any tile volume % 32 == 0
  kTile384 = 1,   // 384 queries per work item (8 waves x 48); tile volume % 384 == 0
};

constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, blocks dispatched round-robin
constexpr int kCusPerXcd = 32;    // compute units per XCD (256 in all)
constexpr int kKeyBlock = 32;     // keys staged in LDS per pipeline step
constexpr int kMaxTileTokens = 4096;

// LDS row strides of the forward kernel's K and V stages (bytes), padded so
// that the MFMA operand reads avoid bank conflicts.  Measured on gfx950 with
// the kernel's own access patterns (16 rows x 16 B per 16-lane group for K,
// 4 rows x 32 B per group for the transposing V reads): a 32-byte pad gives
// the highest LDS throughput for both (154 and 176 B/clk/CU against 111 and
// 129 with a 16-byte pad, 29 and 36 unpadded).
constexpr int fwd_kstride(int head_dim) { return 2 * head_dim + 32; }
constexpr int fwd_vstride(int head_dim) { return 2 * head_dim + 32; }
// Dynamic LDS of a forward launch: two K and two V stages of kKeyBlock keys,
// the tile-local row offsets (tile_tokens ints) and the key-tile base rows of
// the item (max_nkv ints).
constexpr long long fwd_lds_bytes(int head_dim, long long tile_tokens, long long max_nkv) {
  return 2LL * kKeyBlock * (fwd_kstride(head_dim) + fwd_vstride(head_dim)) +
         4LL * (tile_tokens + max_nkv);
}
// Added to it: one word per 32-key step of the longest walk (the steps'
// token-validity words with partial tiles, or the byte offsets of the
// steps' first key rows when K and V are addressed per step).
constexpr long long fwd_lds_step_bytes(long long tile_tokens, long long max_nkv) {
  return 4LL * max_nkv * (tile_tokens / kKeyBlock);
}
constexpr long long kMaxLds = 160 * 1024;

// The backward kernels stream blocks of 32 tokens (keys for dQ, queries for
// dK/dV) through LDS rings of two fp16 tensors with the forward's padded row
// stride: two stages for dQ, three for dK/dV, which also keeps the blocks'
// log-sum-exp and delta rows and two stages of the probability exchange
// between its wave pairs (up to 6 pairs x 2 KiB).  Both keep the tile-local
// row offsets and the item's tile base rows.  The dK/dV layout is the larger.
constexpr int bwd_stride(int head_dim) { return 2 * head_dim + 32; }
// With partial tiles both add one validity word per 32-token block of their
// walk.
constexpr long long bwd_lds_bytes(int head_dim, long long tile_tokens, long long max_list, bool partial) {
  return 3LL * 2 * kKeyBlock * bwd_stride(head_dim) + 3LL * 2 * kKeyBlock * 4 + 2LL * 6 * 2048 +
         4LL * (tile_tokens + max_list) + (partial ? 4LL * max_list * (tile_tokens / kKeyBlock) : 0);
}

struct DeviceTables {
  int32_t *kv_off = nullptr;       // heads*n_tiles + 1
  int32_t *kv_idx = nullptr;       // sum of list lengths
  int32_t *sched = nullptr;        // work items in launch order (-1 = idle)
  int32_t *base_nat = nullptr;     // n_tiles: first token row of each tile, natural order
  int32_t *off_nat = nullptr;      // tile_tokens: row offset of each tile-local token, natural order
  int32_t *base_tm = nullptr;      // n_tiles: tile * tile_tokens
  int32_t *off_tm = nullptr;       // tile_tokens: identity
  int32_t *q_off = nullptr;        // heads*n_tiles + 1
  int32_t *q_idx = nullptr;        // query tiles whose window holds each (head, key tile)
  int32_t *sched_dq = nullptr;     // backward dQ work items in launch order (-1 = idle)
  int32_t *sched_dkdv = nullptr;   // backward dK/dV work items in launch order (-1 = idle)
  int32_t *kmask = nullptr;        // partial plans: n_tiles * tile_tokens/32 validity words
  int32_t *swin = nullptr;         // SWA plans: heads*3 token windows
  int32_t *queue = nullptr;        // dynamic queues: the 8 XCD queues, concatenated
  int32_t *ptab = nullptr;         // split items: 4 per piece (item, first step, end step, group)
  int32_t *gtab = nullptr;         // split items: 2 per group (first piece, piece count)
  int32_t *wlist = nullptr;        // per-work-group lists (codes), and
  int32_t *woff = nullptr;         // their offsets (launch blocks + 1)
  void *block = nullptr;           // the single allocation holding all of the above
  // The upload runs on the stream of the call that made it; `ready` (a
  // hipEvent_t) is recorded after it, and a call on another stream waits
  // for it before its first launch.
  void *upload_stream = nullptr;
  void *ready = nullptr;
};

// Scratch of a forward launch: 16 int32 queue words (the next free entry
// of each of the 9 dynamic queues, the count of finished work groups, an
// "every queue is empty" flag, the count of work items marked for the
// fix-up kernel and the fix-up kernel's finished work groups), one int32
// arrival counter per split item, one bit per work item code (marked:
// redo with V scaled), all zero between launches (the last work group to
// finish, the last piece to arrive and the fix-up kernel reset them); then
// the list of marked items (one int32 per item code), padded to 256 B; then
// one partial-result slot per piece.  A slot holds the piece's unnormalised
// O (QPI x D fp32, in the accumulator layout of the kernel's threads)
// followed by each thread's reference maxima and row-sum partials (2 x QB x
// threads fp32).
constexpr int kQueueWords = 16;
constexpr long long fwd_slot_floats(int head_dim) {
  return 384LL * head_dim + 2LL * 3 * 512;
}
inline long long fwd_bit_words(long long items) { return (items + 31) / 32; }
// int32 words that must be zero before a launch
inline long long fwd_zero_words(long long groups, long long items) {
  return kQueueWords + groups + fwd_bit_words(items);
}
inline long long fwd_counter_bytes(long long groups, long long items) {
  return (4 * (fwd_zero_words(groups, items) + items) + 255) / 256 * 256;
}
inline long long fwd_scratch_bytes(int head_dim, long long groups, long long pieces, long long items) {
  return fwd_counter_bytes(groups, items) + 4LL * fwd_slot_floats(head_dim) * pieces;
}

}  // namespace sta

struct sta_plan {
  int32_t batch = 0, heads = 0, T = 0, H = 0, W = 0, D = 0;
  int32_t tile[3] = {0, 0, 0};
  int32_t grid[3] = {0, 0, 0};
  int32_t V = 0;          // tokens per tile
  // Rows of every 32-key block in the natural layout are the block's first
  // row plus a fixed offset per position in the block (true for tiles whose
  // blocks are whole (t, y) runs of z, e.g. 6x8x8; the tile-major layout
  // always is): the forward then addresses K and V with one per-lane
  // constant and one uniform offset per step.
  bool sep_nat = false;
  int32_t n_tiles = 0;
  int64_t N = 0;          // tokens
  std::vector<int32_t> win;       // heads*3 effective (clamped) windows
  std::vector<int32_t> kv_off;    // heads*n_tiles + 1
  std::vector<int32_t> kv_idx;    // key tiles per (head, query tile), launch order
  std::vector<int32_t> sched;     // launch order of work items, -1 = idle, -2 - p = piece p
  // Work items split by key range (the forward's last, partial round of
  // equal-cost items would otherwise leave most compute units idle): piece
  // p walks steps [ptab[4p+1], ptab[4p+2]) of item ptab[4p] and belongs to
  // group ptab[4p+3]; group g's pieces are ptab entries gtab[2g] ..
  // gtab[2g] + gtab[2g+1] - 1.  The last piece of a group to finish merges
  // the group's partial results (through the launch's scratch).
  std::vector<int32_t> ptab, gtab;
  int32_t n_pieces = 0, n_groups = 0;
  // Dynamic queues (the 384-query forward): per-XCD queues of whole work
  // items and a ninth queue of pieces, concatenated (queue k at
  // queue[qoff[k] .. qoff[k+1])).  A work group takes the next entry of its
  // own XCD's queue with an atomic counter, when that is empty the next
  // entry of another XCD's, and only when every XCD queue is empty a piece,
  // so that XCDs that run faster take more of the work and the pieces fill
  // the end of the launch.  The launch has dyn_blocks work groups (more than
  // entries); those that find every queue empty exit.  dyn_blocks == 0:
  // static launch, work group b runs sched[b].
  std::vector<int32_t> queue;
  int32_t qoff[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  int32_t dyn_blocks = 0;
  // Plans with fewer work items than compute units: the launch's key steps
  // (all items in decreasing-cost order, concatenated) are cut into one
  // contiguous range per compute unit; work group b runs the whole items
  // and pieces of its range, the codes wlist[woff[b] .. woff[b+1]), in
  // turn.  Empty otherwise.
  std::vector<int32_t> wlist, woff;
  std::vector<int32_t> base_nat, off_nat;
  std::vector<int32_t> base_tm, off_tm;   // tile-major layout: tile * V, identity
  int64_t pairs = 0;
  int32_t max_nkv = 0;    // longest key-tile list
  int32_t variant = 0;
  int32_t qpi = 0;        // queries per work item
  int32_t subs = 0;       // work items per (b, head, query tile)
  int64_t items() const { return (int64_t)batch * heads * n_tiles * subs; }   // forward item codes
  long long fwd_scratch() const;                                              // bytes of forward scratch

  // Backward: inverse lists (query tiles whose window holds a key tile) and
  // the schedules of the dQ kernel (items of 32 * bwd_q_waves queries) and
  // the dK/dV kernel (items of 32 * bwd_k_pairs keys).
  std::vector<int32_t> q_off;     // heads*n_tiles + 1
  std::vector<int32_t> q_idx;
  std::vector<int32_t> sched_dq, sched_dkdv;
  int32_t max_nq = 0;     // longest inverse list
  int32_t bwd_q_waves = 0;   // waves per dQ work item
  int32_t bwd_k_pairs = 0;   // wave pairs per dK/dV work item
  int32_t bwd_q_subs = 0, bwd_k_subs = 0;   // work items per (b, head, tile)
  bool bwd_ok = false;    // the backward kernels' LDS fits

  // Partial tiles (an extent that is not a multiple of its tile size):
  // bit i of kmask[tile * V/32 + b] is set iff tile-local token 32b + i
  // exists.  Empty for plans whose tiles are all whole.
  bool partial = false;
  std::vector<int32_t> kmask;

  // Token-wise sliding window attention (a comparison baseline): every query
  // token has its own window of swin[3h..3h+2] tokens (clamped to the
  // extents); tiles only group queries into work items.  No key-tile lists.
  bool swa = false;
  std::vector<int32_t> swin;

  mutable std::mutex mu;
  mutable std::map<int, sta::DeviceTables> dev;   // per HIP device ordinal
  // Forward scratch of plans with split items, one per (device, stream):
  // launches on one stream run in order, so they can share it.
  mutable std::map<std::pair<int, void *>, void *> scratch;
};

namespace sta {

// Host-only plan construction (no HIP calls).  Defined in sta_plan.cpp.
// partial_ok: accept extents that are not multiples of their tile size
// (the last tile of such an axis is partial; forward in natural layout only).
sta_status build_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                      const int *window, int head_dim, bool partial_ok, sta_plan **out);

// Token-wise SWA plan (host only).  Defined in sta_plan.cpp.
sta_status build_swa_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                          const int *window_tokens, int head_dim, sta_plan **out);

// Releases device tables; defined in sta_api.hip (needs HIP).
void release_device_tables(sta_plan *plan);

// Process-wide cache of STA plans for sta_forward (host only; defined in
// sta_plan.cpp).  Callers hold a shared reference, so that clearing the
// cache never frees a plan that a call is still using: the last reference
// destroys it.  Returns nullptr and sets *status when the plan cannot be
// built.
std::shared_ptr<sta_plan> cached_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                                      const int *window, int head_dim, sta_status *status);
void clear_plan_cache();

// Test hook: true when the environment holds STA_TEST_FAIL_ALLOC=1; every
// plan, device-table and scratch allocation of the library then fails with
// STA_ERR_ALLOC.
bool test_fail_alloc();

}  // namespace sta

inline long long sta_plan::fwd_scratch() const {
  return sta::fwd_scratch_bytes(D, n_groups, n_pieces, items());
}
