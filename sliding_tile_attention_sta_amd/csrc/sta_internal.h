// Internal definitions shared by the host plan (sta_plan.cpp) and the HIP
// entry points (sta_api.hip).  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "sta.h"

namespace sta {

// Kernel variants: how many query tokens one work group owns.
enum Variant : int32_t {
  kGeneric = 0,   // 32 queries per work item (2 waves x 16); any tile volume % 32 == 0
  kTile384 = 1,   // 384 queries per work item (8 waves x 48); tile volume % 384 == 0
};

constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, blocks dispatched round-robin
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
constexpr long long kMaxLds = 160 * 1024;

// The backward kernels stream blocks of 32 tokens (keys for dQ, queries for
// dK/dV) through LDS rings of two fp16 tensors with the forward's padded row
// stride: two stages for dQ, three for dK/dV, which also keeps the blocks'
// log-sum-exp and delta rows and two stages of the probability exchange
// between its wave pairs (up to 6 pairs x 2 KiB).  Both keep the tile-local
// row offsets and the item's tile base rows.  The dK/dV layout is the larger.
constexpr int bwd_stride(int head_dim) { return 2 * head_dim + 32; }
constexpr long long bwd_lds_bytes(int head_dim, long long tile_tokens, long long max_list) {
  return 3LL * 2 * kKeyBlock * bwd_stride(head_dim) + 3LL * 2 * kKeyBlock * 4 + 2LL * 6 * 2048 +
         4LL * (tile_tokens + max_list);
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
  void *block = nullptr;           // the single allocation holding all of the above
};

}  // namespace sta

struct sta_plan {
  int32_t batch = 0, heads = 0, T = 0, H = 0, W = 0, D = 0;
  int32_t tile[3] = {0, 0, 0};
  int32_t grid[3] = {0, 0, 0};
  int32_t V = 0;          // tokens per tile
  int32_t n_tiles = 0;
  int64_t N = 0;          // tokens
  std::vector<int32_t> win;       // heads*3 effective (clamped) windows
  std::vector<int32_t> kv_off;    // heads*n_tiles + 1
  std::vector<int32_t> kv_idx;    // key tiles per (head, query tile), launch order
  std::vector<int32_t> sched;     // launch order of work items, -1 = idle
  std::vector<int32_t> base_nat, off_nat;
  int64_t pairs = 0;
  int32_t max_nkv = 0;    // longest key-tile list
  int32_t variant = 0;
  int32_t qpi = 0;        // queries per work item
  int32_t subs = 0;       // work items per (b, head, query tile)

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

}  // namespace sta
