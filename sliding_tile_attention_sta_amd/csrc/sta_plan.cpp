// Host-side planning for Sliding Tile Attention (no HIP calls in this file).
//
// Geometry follows the STA definition ("Fast Video Generation with Sliding
// Tile Attention", arXiv 2502.04507: index page, Abstract; gptget summary
// page, Methodology and Novelty): non-overlapping 3D tiles, a per-head window
// of whole tiles that slides tile by tile.  Readings where the pages are
// silent: windows wider than the grid are clamped to it, and a window is
// centred on its query tile and shifted inward at the borders.

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <functional>
#include <new>
#include <numeric>
#include <queue>

#include "sta_internal.h"

namespace sta {
namespace {

inline int window_start(int c, int w, int n) {
  int s = c - (w - 1) / 2;
  if (s < 0) s = 0;
  if (s > n - w) s = n - w;
  return s;
}

// Work items per XCD queue, in launch order.  Item code ((b * heads + h) *
// n_tiles + t) * subs + sub; its cost is the length of list (h, t) in off.
// Items are sorted by decreasing cost, cut into chunks of consecutive items,
// and each chunk goes to the XCD with the least accumulated cost.  Blocks
// are dispatched to XCDs round-robin (block b runs on XCD b % 8), so XCD x's
// queue is placed at blocks x, x + 8, x + 16, ...  Within an XCD the
// hardware hands blocks to free compute units in order, which is list
// scheduling of a decreasing-cost list.  Chunks keep spatially adjacent
// tiles of one head on the same XCD, whose L2 then serves their overlapping
// windows; launches of fewer items than 8 full chunks use smaller chunks,
// so that every XCD gets work.  The first n_whole items of the order go to
// the queues; *order receives the whole order.
template <typename Off>
std::vector<std::vector<int32_t>> build_queues(const sta_plan *p, const std::vector<Off> &off, int subs,
                                               std::vector<int64_t> *order_out = nullptr,
                                               int64_t n_whole = -1) {
  const int64_t n_items = (int64_t)p->batch * p->heads * p->n_tiles * subs;
  std::vector<int64_t> order(n_items);
  std::iota(order.begin(), order.end(), 0);
  auto cost = [&](int64_t code) {
    int64_t rest = code / subs;
    int t = (int)(rest % p->n_tiles);
    int h = (int)((rest / p->n_tiles) % p->heads);
    return (int64_t)off[(size_t)h * p->n_tiles + t + 1] - off[(size_t)h * p->n_tiles + t];
  };
  // ties: by (batch, head), then the tile's Morton (Z-order) code, so that
  // a chunk of consecutive items (the ones an XCD runs at once) is a compact
  // block of tiles whose windows overlap, and the work groups of an XCD
  // read the same key/value blocks from its L2 at about the same step
  // (a raster run of 32 tiles spans twice the key tiles of a 2x4x4 block)
  const int nH = p->grid[1], nW = p->grid[2];
  auto morton = [&](int t) {
    const uint32_t c[3] = {(uint32_t)(t / (nH * nW)), (uint32_t)((t / nW) % nH), (uint32_t)(t % nW)};
    uint64_t m = 0;
    for (int b = 0; b < 16; ++b)
      for (int d = 0; d < 3; ++d) m |= (uint64_t)((c[d] >> b) & 1u) << (3 * b + (2 - d));
    return m;
  };
  std::vector<uint64_t> mk((size_t)p->n_tiles);
  for (int t = 0; t < p->n_tiles; ++t) mk[t] = morton(t);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    const int64_t ca = cost(a), cb = cost(b);
    if (ca != cb) return ca > cb;
    const int64_t ra = a / subs, rb = b / subs;
    const int64_t ga = ra / p->n_tiles, gb = rb / p->n_tiles;
    if (ga != gb) return ga < gb;
    const uint64_t ma = mk[ra % p->n_tiles], mb = mk[rb % p->n_tiles];
    if (ma != mb) return ma < mb;
    return a < b;
  });
  if (n_whole < 0) n_whole = n_items;
  const int64_t chunk = std::max<int64_t>(1, std::min<int64_t>(kCusPerXcd, (n_whole + kXcds - 1) / kXcds));
  std::vector<std::vector<int32_t>> queue(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (int64_t i = 0; i < n_whole; i += chunk) {
    int64_t end = std::min(n_whole, i + chunk);
    int64_t c = 0;
    for (int64_t j = i; j < end; ++j) c += cost(order[j]);
    int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += c;
    for (int64_t j = i; j < end; ++j) queue[x].push_back((int32_t)order[j]);
  }
  if (order_out) order_out->swap(order);
  return queue;
}

std::vector<int32_t> interleave(const std::vector<std::vector<int32_t>> &queue) {
  size_t len = 0;
  for (auto &q : queue) len = std::max(len, q.size());
  std::vector<int32_t> sched(len * kXcds, -1);
  for (int x = 0; x < kXcds; ++x)
    for (size_t s = 0; s < queue[x].size(); ++s) sched[s * kXcds + x] = queue[x][s];
  return sched;
}

constexpr int64_t kMaxPieces = 512;
constexpr int64_t kMinPieceSteps = 32;

// The forward's dynamic queues (see sta_plan::queue): per-XCD queues of
// whole work items, and a ninth queue of the pieces of split items, which
// work groups take only once every XCD queue is empty.  Work items are
// coarse: one 720p item is about 1/28 of a compute unit's share of the
// launch, so without pieces the units that drew the last items run up to a
// whole item after the others.  Splitting (split = true): the last R items
// of the decreasing-cost order are cut into k pieces of consecutive key
// steps (steps_per_entry per list entry; boundaries on multiples of align
// steps), R = 64 (a quarter of the chip's compute units), k = 4, fewer if a
// piece would walk less than 32 steps or there would be more than 512
// pieces, and no split at k < 2.  With fewer items than compute units,
// either one contiguous range of key steps per compute unit (per-work-group
// lists, sta_plan::wlist, where that pays by more than kRangeOverheadSteps)
// or every item into the k whose pieces take the fewest rounds of the chip.
// Measured on MI355X with the 7,200 equal items of the 720p workload: 64
// items in 4 pieces ran 1 % faster than no split; 128 or 256 items in 4
// pieces less so, and 256 in 8 slower than no split (every piece adds the
// write of its partial result, two fences and its share of the merge).
//
// A range pays only if it saves more than this many 32-key steps against
// one round of whole items (measured on MI355X: see build_forward_queues).
constexpr int64_t kRangeOverheadSteps = 32;
// Per-unit ranges need at least units / this many items.  12x24x24 with one
// head (18 items, about 15 ranges each) ran 3.5 % slower in ranges than in
// the 4-way split below; with two heads (36 items, about 7 ranges each)
// 2.6 % faster (MI355X, one session).
constexpr int64_t kMaxRangesPerItem = 8;

template <typename Off>
void build_forward_queues(sta_plan *p, const std::vector<Off> &off, int64_t steps_per_entry, int64_t align,
                          bool split) {
  std::vector<int64_t> order;
  auto whole = build_queues(p, off, p->subs, &order);
  const int64_t n_items = (int64_t)order.size();
  auto steps = [&](int64_t code) {
    const int64_t rest = code / p->subs;
    const int t = (int)(rest % p->n_tiles), h = (int)((rest / p->n_tiles) % p->heads);
    return ((int64_t)off[(size_t)h * p->n_tiles + t + 1] - off[(size_t)h * p->n_tiles + t]) * steps_per_entry;
  };
  const int64_t units = kXcds * kCusPerXcd;
  int64_t total_steps = 0, max_steps = 0;
  for (int64_t i = 0; i < n_items; ++i) {
    total_steps += steps(order[i]);
    max_steps = std::max(max_steps, steps(order[i]));
  }
  if (split && n_items * kMaxRangesPerItem >= units && n_items < units &&
      total_steps + kRangeOverheadSteps * units < max_steps * units) {
    // Fewer items than compute units (but not so few that an item spans
    // more than about kMaxRangesPerItem ranges, whose partial results its
    // last piece would read back), and one range of the launch's key steps
    // per compute unit beats one round of whole items by more than a
    // range's overhead (its pieces' publication and merge, and a second
    // item's prologue): the ranges are contiguous (boundaries on multiples
    // of align steps), so every unit walks the same number of steps (within
    // align).  12x24x24's 144 items of 216 steps: 121.5 steps per unit
    // against two rounds of 72-step pieces; one round of 192 items of 108
    // steps stays whole (81 steps per range ran 5 % slower on MI355X).  An
    // item inside one range runs whole; an item cut by range boundaries
    // becomes a group of pieces that merge as in the tail split.  Ranges 32
    // apart go to the same XCD (range u to block (u mod 32) * 8 + u / 32,
    // blocks being dispatched to XCDs round-robin), so ranges that share an
    // item share an L2.
    std::vector<int64_t> start(n_items + 1, 0);
    for (int64_t i = 0; i < n_items; ++i) start[i + 1] = start[i] + steps(order[i]) / align;
    const int64_t total = start[n_items];
    std::vector<std::vector<std::pair<int64_t, int64_t>>> cut(n_items);   // (lo, hi) per item
    std::vector<std::vector<std::pair<int64_t, int64_t>>> unit_of(n_items);   // (unit, piece slot)
    int64_t it = 0;
    for (int64_t u = 0; u < units; ++u) {
      int64_t lo = total * u / units;
      const int64_t hi = total * (u + 1) / units;
      while (lo < hi) {
        while (start[it + 1] <= lo) ++it;
        const int64_t e = std::min(hi, start[it + 1]);
        unit_of[it].push_back({u, (int64_t)cut[it].size()});
        cut[it].push_back({lo - start[it], e - start[it]});
        lo = e;
      }
    }
    std::vector<std::vector<int32_t>> codes(units);
    for (int64_t i = 0; i < n_items; ++i) {
      if (cut[i].size() == 1) {
        codes[unit_of[i][0].first].push_back((int32_t)order[i]);
        continue;
      }
      const int32_t group = p->n_groups++;
      p->gtab.push_back(p->n_pieces);
      p->gtab.push_back((int32_t)cut[i].size());
      for (size_t j = 0; j < cut[i].size(); ++j) {
        p->ptab.push_back((int32_t)order[i]);
        p->ptab.push_back((int32_t)(cut[i][j].first * align));
        p->ptab.push_back((int32_t)(cut[i][j].second * align));
        p->ptab.push_back(group);
        codes[unit_of[i][j].first].push_back(-2 - p->n_pieces++);
      }
    }
    p->woff.assign(units + 1, 0);
    p->wlist.clear();
    for (int64_t b = 0; b < units; ++b) {
      const int64_t u = (b % kXcds) * kCusPerXcd + b / kXcds;
      p->wlist.insert(p->wlist.end(), codes[u].begin(), codes[u].end());
      p->woff[b + 1] = (int32_t)p->wlist.size();
    }
    p->sched = p->wlist;
    p->queue.clear();
    for (int x = 0; x < 10; ++x) p->qoff[x] = 0;
    p->dyn_blocks = 0;
    return;
  }
  int64_t best_r = 0;
  int best_k = 1;
  if (split && n_items > 0) {
    best_r = n_items < units ? n_items : units / 4;
    int kmax = (int)std::min<int64_t>(4, kMaxPieces / best_r);
    for (int64_t i = n_items - best_r; i < n_items; ++i)   // the cheapest items
      kmax = (int)std::min<int64_t>(kmax, steps(order[i]) / align / std::max<int64_t>(1, kMinPieceSteps / align));
    if (n_items >= units) {
      best_k = kmax;
    } else {
      // Fewer items than compute units: the k (<= kmax) whose pieces take
      // the fewest rounds of the chip, ceil(n k / units) / k, ties to the
      // smaller k.
      double best = 1.0;
      for (int k = 2; k <= kmax; ++k) {
        const double t = (double)((n_items * k + units - 1) / units) / k;
        if (t < best - 1e-9) { best = t; best_k = k; }
      }
    }
    if (best_k < 2) { best_r = 0; best_k = 1; }
  }
  if (best_r > 0) whole = build_queues(p, off, p->subs, nullptr, n_items - best_r);
  std::vector<int32_t> pieces;
  for (int64_t i = n_items - best_r; i < n_items; ++i) {
    const int64_t u = steps(order[i]) / align;
    const int32_t group = p->n_groups++;
    p->gtab.push_back(p->n_pieces);
    p->gtab.push_back(best_k);
    for (int j = 0; j < best_k; ++j) {
      p->ptab.push_back((int32_t)order[i]);
      p->ptab.push_back((int32_t)(u * j / best_k * align));
      p->ptab.push_back((int32_t)(u * (j + 1) / best_k * align));
      p->ptab.push_back(group);
      pieces.push_back(-2 - p->n_pieces++);
    }
  }
  // sched: the XCD queues interleaved, then the pieces.
  p->sched = interleave(whole);
  p->sched.insert(p->sched.end(), pieces.begin(), pieces.end());
  // Launch: 1/16 more work groups per XCD than its queue holds (at least 8
  // more), so that an XCD whose units run faster can take entries from the
  // others' queues, plus the pieces spread over the XCDs.
  size_t len = 0;
  p->queue.clear();
  p->qoff[0] = 0;
  for (int x = 0; x < kXcds; ++x) {
    p->queue.insert(p->queue.end(), whole[x].begin(), whole[x].end());
    p->qoff[x + 1] = (int32_t)p->queue.size();
    len = std::max(len, whole[x].size());
  }
  p->queue.insert(p->queue.end(), pieces.begin(), pieces.end());
  p->qoff[kXcds + 1] = (int32_t)p->queue.size();
  len += (pieces.size() + kXcds - 1) / kXcds;
  p->dyn_blocks = (int32_t)(kXcds * (len + std::max<size_t>(8, len / 16)));
}

template <typename Off>
std::vector<int32_t> build_schedule(sta_plan *p, const std::vector<Off> &off, int subs) {
  return interleave(build_queues(p, off, subs));
}

}  // namespace

sta_status build_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                      const int *window, int head_dim, bool partial_ok, sta_plan **out) {
  if (!out || !tile || !window) return STA_ERR_ARG;
  *out = nullptr;
  if (batch < 1 || heads < 1 || T < 1 || H < 1 || W < 1) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (tile[d] < 1) return STA_ERR_ARG;
  for (int i = 0; i < heads * 3; ++i)
    if (window[i] < 1) return STA_ERR_ARG;
  const int ext[3] = {T, H, W};
  for (int d = 0; d < 3; ++d)
    if (ext[d] % tile[d] != 0 && !partial_ok) return STA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return STA_ERR_UNSUPPORTED;
  const int64_t V64 = (int64_t)tile[0] * tile[1] * tile[2];
  if (V64 % kKeyBlock != 0 || V64 > kMaxTileTokens) return STA_ERR_UNSUPPORTED;
  const int64_t N64 = (int64_t)T * H * W;
  // Element offsets are 64-bit in the kernels; token rows and table entries are int32.
  if (N64 * batch * heads > (int64_t)INT32_MAX) return STA_ERR_UNSUPPORTED;
  // Size checks before any list is built.  Every clamped window holds the
  // same number of key tiles for each query tile of its head.  The lists of
  // all heads sit in one table indexed by int32 offsets (as do their
  // inverses, which hold as many entries), and the longest list must fit the
  // forward kernel's LDS beside its K/V stages.
  {
    int64_t grid[3], pairs = 0, longest = 0;
    bool partial = false;
    for (int d = 0; d < 3; ++d) {
      grid[d] = (ext[d] + tile[d] - 1) / tile[d];
      partial |= ext[d] % tile[d] != 0;
    }
    const int64_t n_tiles = grid[0] * grid[1] * grid[2];
    for (int h = 0; h < heads && pairs <= (int64_t)INT32_MAX; ++h) {
      int64_t vol = 1;
      for (int d = 0; d < 3; ++d) vol *= std::min<int64_t>(window[h * 3 + d], grid[d]);
      longest = std::max(longest, vol);
      pairs += n_tiles * vol;
    }
    if (pairs > (int64_t)INT32_MAX) return STA_ERR_UNSUPPORTED;
    if (fwd_lds_bytes(head_dim, V64, longest) + (partial ? fwd_lds_step_bytes(V64, longest) : 0) > kMaxLds)
      return STA_ERR_UNSUPPORTED;
  }

  sta_plan *p = new (std::nothrow) sta_plan();
  if (!p) return STA_ERR_ALLOC;
  try {
    if (test_fail_alloc()) throw std::bad_alloc();
    p->batch = batch; p->heads = heads; p->T = T; p->H = H; p->W = W; p->D = head_dim;
    for (int d = 0; d < 3; ++d) {
      p->tile[d] = tile[d];
      p->grid[d] = (ext[d] + tile[d] - 1) / tile[d];
      if (ext[d] % tile[d] != 0) p->partial = true;
    }
    p->V = (int32_t)V64;
    p->N = N64;
    p->n_tiles = p->grid[0] * p->grid[1] * p->grid[2];
    if (p->V % 384 == 0) {
      p->variant = kTile384; p->qpi = 384;
    } else {
      p->variant = kGeneric; p->qpi = 32;
    }
    p->subs = p->V / p->qpi;

    // Per-head clamped windows and per-(head, query tile) key-tile lists.
    // Launch order inside a window: raster order of (a mod wT, b mod wH,
    // c mod wW).  The map from a tile coordinate to its residue is one-to-one
    // on any w consecutive tiles, so query tiles whose windows overlap visit
    // their shared key tiles at the same step, which the L2 rewards.
    p->win.resize(heads * 3);
    p->kv_off.assign((size_t)heads * p->n_tiles + 1, 0);
    const int nT = p->grid[0], nH = p->grid[1], nW = p->grid[2];
    for (int h = 0; h < heads; ++h) {
      int w[3];
      for (int d = 0; d < 3; ++d) w[d] = std::min(window[h * 3 + d], p->grid[d]);
      for (int d = 0; d < 3; ++d) p->win[h * 3 + d] = w[d];
      for (int qt = 0; qt < p->n_tiles; ++qt) {
        const int ct = qt / (nH * nW), cy = (qt / nW) % nH, cz = qt % nW;
        const int st = window_start(ct, w[0], nT), sy = window_start(cy, w[1], nH),
                  sz = window_start(cz, w[2], nW);
        for (int rt = 0; rt < w[0]; ++rt)
          for (int ry = 0; ry < w[1]; ++ry)
            for (int rz = 0; rz < w[2]; ++rz) {
              // the tile in [s, s + w) whose coordinate is congruent to r mod w
              const int a = st + ((rt - st % w[0]) % w[0] + w[0]) % w[0];
              const int b = sy + ((ry - sy % w[1]) % w[1] + w[1]) % w[1];
              const int c = sz + ((rz - sz % w[2]) % w[2] + w[2]) % w[2];
              p->kv_idx.push_back((a * nH + b) * nW + c);
            }
        p->kv_off[(size_t)h * p->n_tiles + qt + 1] = (int32_t)p->kv_idx.size();
      }
    }
    p->pairs = (int64_t)p->kv_idx.size();
    for (size_t i = 0; i + 1 < p->kv_off.size(); ++i)
      p->max_nkv = std::max(p->max_nkv, p->kv_off[i + 1] - p->kv_off[i]);
    // The forward kernel keeps two K and two V stages of 32 keys plus the
    // tile-local row offsets and the item's key-tile rows in LDS (160 KiB).
    if (fwd_lds_bytes(head_dim, p->V, p->max_nkv) + (p->partial ? fwd_lds_step_bytes(p->V, p->max_nkv) : 0) >
        kMaxLds) {
      delete p;
      return STA_ERR_UNSUPPORTED;
    }

    // Token row tables for the natural layout.
    p->base_nat.resize(p->n_tiles);
    for (int qt = 0; qt < p->n_tiles; ++qt) {
      const int ct = qt / (nH * nW), cy = (qt / nW) % nH, cz = qt % nW;
      p->base_nat[qt] = ((ct * tile[0]) * H + cy * tile[1]) * W + cz * tile[2];
    }
    p->off_nat.resize(p->V);
    for (int j = 0; j < p->V; ++j) {
      const int lt = j / (tile[1] * tile[2]), ly = (j / tile[2]) % tile[1], lz = j % tile[2];
      p->off_nat[j] = (lt * H + ly) * W + lz;
    }
    p->base_tm.resize(p->n_tiles);
    for (int qt = 0; qt < p->n_tiles; ++qt) p->base_tm[qt] = qt * p->V;
    p->off_tm.resize(p->V);
    std::iota(p->off_tm.begin(), p->off_tm.end(), 0);
    p->sep_nat = true;
    for (int j = 0; j < p->V; ++j)
      if (p->off_nat[j] - p->off_nat[j / kKeyBlock * kKeyBlock] != p->off_nat[j % kKeyBlock] - p->off_nat[0])
        p->sep_nat = false;
    if (p->partial) {
      // Token validity per tile; with partial tiles base + off can name a
      // row past the tile's edge (or past the tensor), which the kernel
      // clamps and masks.
      p->kmask.assign((size_t)p->n_tiles * (p->V / 32), 0);
      for (int t = 0; t < p->n_tiles; ++t) {
        const int ct = t / (nH * nW), cy = (t / nW) % nH, cz = t % nW;
        for (int j = 0; j < p->V; ++j) {
          const int lt = j / (tile[1] * tile[2]), ly = (j / tile[2]) % tile[1], lz = j % tile[2];
          if (ct * tile[0] + lt < T && cy * tile[1] + ly < H && cz * tile[2] + lz < W)
            p->kmask[(size_t)t * (p->V / 32) + j / 32] |= (int32_t)(1u << (j % 32));
        }
      }
    }
    // Split items need the 384-query kernel.  Every piece's first key block
    // must hold an existing key (its reference maximum comes from it): with
    // partial tiles, pieces start on key-tile boundaries (a tile's first
    // token always exists).
    if (p->variant == kTile384)
      build_forward_queues(p, p->kv_off, p->V / kKeyBlock, p->partial ? p->V / kKeyBlock : 1, true);
    else
      p->sched = build_schedule(p, p->kv_off, p->subs);

    // Backward: the inverse of the key-tile lists (query tiles whose window
    // holds the key tile), per head, and the two backward schedules.  Launch
    // order inside a list: by (a mod wT, b mod wH, c mod wW) as for the key
    // tiles, ties in raster order.  Away from the borders a key tile is seen
    // by w consecutive query tiles per axis, so key tiles that share query
    // tiles visit them at the same step.
    p->q_off.assign((size_t)heads * p->n_tiles + 1, 0);
    {
      // Query tiles are visited in (residue, raster) order and appended to
      // the lists of their key tiles, so every list comes out in that order.
      std::vector<std::vector<int32_t>> inv(p->n_tiles);
      std::vector<int32_t> res(p->n_tiles), by_res(p->n_tiles);
      for (int h = 0; h < heads; ++h) {
        for (auto &v : inv) v.clear();
        const int *w = &p->win[h * 3];
        for (int t = 0; t < p->n_tiles; ++t) {
          const int ct = t / (nH * nW), cy = (t / nW) % nH, cz = t % nW;
          res[t] = ((ct % w[0]) * w[1] + cy % w[1]) * w[2] + cz % w[2];
        }
        std::iota(by_res.begin(), by_res.end(), 0);
        std::stable_sort(by_res.begin(), by_res.end(), [&](int32_t x, int32_t y) { return res[x] < res[y]; });
        for (const int32_t qt : by_res) {
          const size_t i = (size_t)h * p->n_tiles + qt;
          for (int32_t e = p->kv_off[i]; e < p->kv_off[i + 1]; ++e) inv[p->kv_idx[e]].push_back(qt);
        }
        for (int kt = 0; kt < p->n_tiles; ++kt) {
          p->q_idx.insert(p->q_idx.end(), inv[kt].begin(), inv[kt].end());
          p->q_off[(size_t)h * p->n_tiles + kt + 1] = (int32_t)p->q_idx.size();
          p->max_nq = std::max(p->max_nq, (int32_t)inv[kt].size());
        }
      }
    }
    p->bwd_q_waves = p->V % 128 == 0 ? 4 : 1;
    p->bwd_k_pairs = p->V % 192 == 0 ? 6 : p->V % 128 == 0 ? 4 : 1;
    p->bwd_q_subs = p->V / (32 * p->bwd_q_waves);
    p->bwd_k_subs = p->V / (32 * p->bwd_k_pairs);
    p->bwd_ok = bwd_lds_bytes(head_dim, p->V, std::max(p->max_nkv, p->max_nq), p->partial) <= kMaxLds;
    if (p->bwd_ok) {
      p->sched_dq = build_schedule(p, p->kv_off, p->bwd_q_subs);
      p->sched_dkdv = build_schedule(p, p->q_off, p->bwd_k_subs);
    }
  } catch (const std::bad_alloc &) {
    delete p;
    return STA_ERR_ALLOC;
  }
  *out = p;
  return STA_OK;
}

sta_status build_swa_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                          const int *window_tokens, int head_dim, sta_plan **out) {
  if (!out || !tile || !window_tokens) return STA_ERR_ARG;
  *out = nullptr;
  if (batch < 1 || heads < 1 || T < 1 || H < 1 || W < 1) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (tile[d] < 1) return STA_ERR_ARG;
  for (int i = 0; i < heads * 3; ++i)
    if (window_tokens[i] < 1) return STA_ERR_ARG;
  const int ext[3] = {T, H, W};
  for (int d = 0; d < 3; ++d)
    if (ext[d] % tile[d] != 0) return STA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return STA_ERR_UNSUPPORTED;
  const int64_t V64 = (int64_t)tile[0] * tile[1] * tile[2];
  if (V64 % kKeyBlock != 0 || V64 > kMaxTileTokens) return STA_ERR_UNSUPPORTED;
  const int64_t N64 = (int64_t)T * H * W;
  if (N64 * batch * heads > (int64_t)INT32_MAX) return STA_ERR_UNSUPPORTED;
  if (fwd_lds_bytes(head_dim, V64, 0) > kMaxLds) return STA_ERR_UNSUPPORTED;

  sta_plan *p = new (std::nothrow) sta_plan();
  if (!p) return STA_ERR_ALLOC;
  try {
    if (test_fail_alloc()) throw std::bad_alloc();
    p->batch = batch; p->heads = heads; p->T = T; p->H = H; p->W = W; p->D = head_dim;
    for (int d = 0; d < 3; ++d) { p->tile[d] = tile[d]; p->grid[d] = ext[d] / tile[d]; }
    p->V = (int32_t)V64;
    p->N = N64;
    p->n_tiles = p->grid[0] * p->grid[1] * p->grid[2];
    p->swa = true;
    if (p->V % 384 == 0) {
      p->variant = kTile384; p->qpi = 384;
    } else {
      p->variant = kGeneric; p->qpi = 32;
    }
    p->subs = p->V / p->qpi;
    p->swin.resize((size_t)heads * 3);
    p->win.resize((size_t)heads * 3);
    for (int h = 0; h < heads; ++h)
      for (int d = 0; d < 3; ++d) p->swin[h * 3 + d] = p->win[h * 3 + d] = std::min(window_tokens[h * 3 + d], ext[d]);
    // Work per (head, query tile): rows (t, y) of the union of the tile's
    // query windows times the 32-key runs covering its z range.
    auto start = [](int x, int w, int e) { return std::min(std::max(x - (w - 1) / 2, 0), e - w); };
    std::vector<int64_t> cost_off((size_t)heads * p->n_tiles + 1, 0);
    const int nH = p->grid[1], nW = p->grid[2];
    for (int h = 0; h < heads; ++h)
      for (int qt = 0; qt < p->n_tiles; ++qt) {
        const int c[3] = {qt / (nH * nW), (qt / nW) % nH, qt % nW};
        int64_t span[3];
        for (int d = 0; d < 3; ++d) {
          const int w = p->swin[h * 3 + d];
          const int lo = start(c[d] * tile[d], w, ext[d]);
          const int hi = start(c[d] * tile[d] + tile[d] - 1, w, ext[d]) + w;
          span[d] = hi - lo;
        }
        const int64_t steps = span[0] * span[1] * ((span[2] + kKeyBlock - 1) / kKeyBlock);
        cost_off[(size_t)h * p->n_tiles + qt + 1] = cost_off[(size_t)h * p->n_tiles + qt] + steps;
      }
    p->kv_off.assign((size_t)heads * p->n_tiles + 1, 0);
    p->q_off.assign((size_t)heads * p->n_tiles + 1, 0);
    p->base_nat.resize(p->n_tiles);
    for (int qt = 0; qt < p->n_tiles; ++qt) {
      const int ct = qt / (nH * nW), cy = (qt / nW) % nH, cz = qt % nW;
      p->base_nat[qt] = ((ct * tile[0]) * H + cy * tile[1]) * W + cz * tile[2];
    }
    p->off_nat.resize(p->V);
    for (int j = 0; j < p->V; ++j) {
      const int lt = j / (tile[1] * tile[2]), ly = (j / tile[2]) % tile[1], lz = j % tile[2];
      p->off_nat[j] = (lt * H + ly) * W + lz;
    }
    p->base_tm.resize(p->n_tiles);
    for (int qt = 0; qt < p->n_tiles; ++qt) p->base_tm[qt] = qt * p->V;
    p->off_tm.resize(p->V);
    std::iota(p->off_tm.begin(), p->off_tm.end(), 0);
    if (p->variant == kTile384)
      build_forward_queues(p, cost_off, 1, 1, false);
    else
      p->sched = build_schedule(p, cost_off, p->subs);
  } catch (const std::bad_alloc &) {
    delete p;
    return STA_ERR_ALLOC;
  }
  *out = p;
  return STA_OK;
}

// The n entries at src in ascending order, the first cap of them written to
// out (no allocation: the query entry points never throw).
sta_status sorted_list(const int32_t *src, int32_t n, int32_t *out, int cap, int *count) {
  *count = n;
  if (!out && cap > 0) return STA_ERR_ARG;
  if (cap > 0) std::partial_sort_copy(src, src + n, out, out + std::min(cap, n));
  return n > cap ? STA_ERR_ARG : STA_OK;
}

bool test_fail_alloc() {
  const char *e = std::getenv("STA_TEST_FAIL_ALLOC");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

namespace {
std::mutex g_cache_mu;
std::map<std::vector<int>, std::shared_ptr<sta_plan>> g_cache;
}  // namespace

std::shared_ptr<sta_plan> cached_plan(int batch, int heads, int T, int H, int W, const int tile[3],
                                      const int *window, int head_dim, sta_status *status) {
  *status = STA_OK;
  if (!tile || !window || heads < 1) {
    *status = STA_ERR_ARG;
    return nullptr;
  }
  try {
    std::vector<int> key = {batch, heads, T, H, W, tile[0], tile[1], tile[2], head_dim};
    key.insert(key.end(), window, window + 3 * (size_t)heads);
    std::lock_guard<std::mutex> lock(g_cache_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
    sta_plan *p = nullptr;
    // extents that are not multiples of the tile: a plan with partial tiles
    *status = build_plan(batch, heads, T, H, W, tile, window, head_dim, true, &p);
    if (*status != STA_OK) return nullptr;
    // (if the shared state cannot be allocated, the constructor destroys p)
    std::shared_ptr<sta_plan> sp(p, [](sta_plan *x) { sta_plan_destroy(x); });
    g_cache.emplace(std::move(key), sp);
    return sp;
  } catch (const std::bad_alloc &) {
    *status = STA_ERR_ALLOC;
    return nullptr;
  }
}

void clear_plan_cache() {
  std::map<std::vector<int>, std::shared_ptr<sta_plan>> old;
  {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    old.swap(g_cache);
  }
  // the cache's references are dropped here, outside the lock; a plan still
  // in use by a call is destroyed when that call releases it
}

}  // namespace sta

extern "C" {

sta_status sta_clear_plan_cache(void) {
  sta::clear_plan_cache();
  return STA_OK;
}

sta_status sta_swa_plan_create(int batch, int heads, int T, int H, int W, const int tile[3],
                               const int *window_tokens, int head_dim, sta_plan **out) {
  return sta::build_swa_plan(batch, heads, T, H, W, tile, window_tokens, head_dim, out);
}

sta_status sta_plan_create(int batch, int heads, int T, int H, int W, const int tile[3],
                           const int *window, int head_dim, sta_plan **out) {
  return sta::build_plan(batch, heads, T, H, W, tile, window, head_dim, false, out);
}

sta_status sta_plan_create_ex(int batch, int heads, int T, int H, int W, const int tile[3],
                              const int *window, int head_dim, int flags, sta_plan **out) {
  if (flags & ~STA_PLAN_PARTIAL_TILES) return STA_ERR_ARG;
  return sta::build_plan(batch, heads, T, H, W, tile, window, head_dim,
                         (flags & STA_PLAN_PARTIAL_TILES) != 0, out);
}

sta_status sta_plan_destroy(sta_plan *plan) {
  if (!plan) return STA_OK;
  sta::release_device_tables(plan);
  delete plan;
  return STA_OK;
}

sta_status sta_plan_get_info(const sta_plan *p, sta_plan_info *info) {
  if (!p || !info) return STA_ERR_ARG;
  std::memset(info, 0, sizeof(*info));
  info->batch = p->batch; info->heads = p->heads;
  info->T = p->T; info->H = p->H; info->W = p->W; info->head_dim = p->D;
  for (int d = 0; d < 3; ++d) { info->tile[d] = p->tile[d]; info->grid[d] = p->grid[d]; }
  info->tile_tokens = p->V;
  info->n_tiles = p->n_tiles;
  info->tokens = p->N;
  info->pairs = p->pairs;
  info->flops = 4.0 * (double)p->V * (double)p->V * (double)p->D * (double)p->pairs * p->batch;
  if (p->swa) {
    // permitted (query, key) pairs only: every query sees prod(w') keys
    double keys = 0.0;
    for (int h = 0; h < p->heads; ++h)
      keys += (double)p->swin[h * 3] * p->swin[h * 3 + 1] * p->swin[h * 3 + 2];
    info->flops = 4.0 * (double)p->N * keys * p->D * p->batch;
  }
  info->swa = p->swa ? 1 : 0;
  info->work_items = (int64_t)p->sched.size();
  info->queries_per_item = p->qpi;
  info->kernel_variant = p->variant;
  info->bwd_supported = p->bwd_ok ? 1 : 0;
  info->bwd_queries_per_item = 32 * p->bwd_q_waves;
  info->bwd_keys_per_item = 32 * p->bwd_k_pairs;
  info->bwd_items_dq = (int64_t)p->sched_dq.size();
  info->bwd_items_dkdv = (int64_t)p->sched_dkdv.size();
  info->partial_tiles = p->partial ? 1 : 0;
  info->split_items = p->n_groups;
  info->pieces = p->n_pieces;
  info->scratch_bytes = p->fwd_scratch();
  info->launch_blocks = p->dyn_blocks ? p->dyn_blocks
                        : !p->woff.empty() ? (int64_t)p->woff.size() - 1
                                           : (int64_t)p->sched.size();
  return STA_OK;
}

sta_status sta_plan_perm(const sta_plan *p, int32_t *perm, int64_t cap) {
  if (!p || !perm || cap < p->N) return STA_ERR_ARG;
  if (p->partial || p->swa) return STA_ERR_UNSUPPORTED;
  for (int qt = 0; qt < p->n_tiles; ++qt)
    for (int j = 0; j < p->V; ++j) perm[(int64_t)qt * p->V + j] = p->base_nat[qt] + p->off_nat[j];
  return STA_OK;
}

sta_status sta_plan_kv_tiles(const sta_plan *p, int head, int q_tile, int32_t *out, int cap,
                             int *count) {
  if (!p || !count || head < 0 || head >= p->heads || q_tile < 0 || q_tile >= p->n_tiles)
    return STA_ERR_ARG;
  const size_t i = (size_t)head * p->n_tiles + q_tile;
  return sta::sorted_list(p->kv_idx.data() + p->kv_off[i], p->kv_off[i + 1] - p->kv_off[i], out, cap, count);
}

sta_status sta_plan_q_tiles(const sta_plan *p, int head, int kv_tile, int32_t *out, int cap,
                            int *count) {
  if (!p || !count || head < 0 || head >= p->heads || kv_tile < 0 || kv_tile >= p->n_tiles)
    return STA_ERR_ARG;
  const size_t i = (size_t)head * p->n_tiles + kv_tile;
  return sta::sorted_list(p->q_idx.data() + p->q_off[i], p->q_off[i + 1] - p->q_off[i], out, cap, count);
}

sta_status sta_plan_walk(const sta_plan *p, int which, int head, int tile, int32_t *out, int cap, int *count) {
  if (!p || !count || (which != 0 && which != 1) || head < 0 || head >= p->heads || tile < 0 ||
      tile >= p->n_tiles || p->swa)
    return STA_ERR_ARG;
  const std::vector<int32_t> &off = which == 0 ? p->kv_off : p->q_off;
  const std::vector<int32_t> &idx = which == 0 ? p->kv_idx : p->q_idx;
  if (off.empty()) return STA_ERR_ARG;
  const size_t i = (size_t)head * p->n_tiles + tile;
  const int n = off[i + 1] - off[i];
  *count = n;
  if (!out && cap > 0) return STA_ERR_ARG;
  for (int j = 0; j < cap && j < n; ++j) out[j] = idx[(size_t)off[i] + j];
  return n > cap ? STA_ERR_ARG : STA_OK;
}

sta_status sta_plan_schedule_bwd(const sta_plan *p, int which, int32_t *out, int64_t cap,
                                 int64_t *count) {
  if (!p || !count || (which != 0 && which != 1)) return STA_ERR_ARG;
  const std::vector<int32_t> &s = which == 0 ? p->sched_dq : p->sched_dkdv;
  *count = (int64_t)s.size();
  if (cap < *count || (!out && *count > 0)) return STA_ERR_ARG;
  if (!s.empty()) std::memcpy(out, s.data(), s.size() * sizeof(int32_t));
  return STA_OK;
}

sta_status sta_plan_pieces(const sta_plan *p, int32_t *out, int64_t cap, int64_t *count) {
  if (!p || !count) return STA_ERR_ARG;
  *count = (int64_t)p->n_pieces;
  if (cap < *count || (!out && *count > 0)) return STA_ERR_ARG;
  for (int32_t i = 0; i < p->n_pieces; ++i) {
    const int32_t g = p->ptab[4 * i + 3];
    out[5 * i + 0] = p->ptab[4 * i + 0];
    out[5 * i + 1] = p->ptab[4 * i + 1];
    out[5 * i + 2] = p->ptab[4 * i + 2];
    out[5 * i + 3] = g;
    out[5 * i + 4] = p->gtab[2 * g + 1];
  }
  return STA_OK;
}

sta_status sta_plan_schedule(const sta_plan *p, int32_t *out, int64_t cap, int64_t *count) {
  if (!p || !count) return STA_ERR_ARG;
  *count = (int64_t)p->sched.size();
  if (cap < *count || !out) return STA_ERR_ARG;
  std::memcpy(out, p->sched.data(), p->sched.size() * sizeof(int32_t));
  return STA_OK;
}

sta_status sta_plan_group_lists(const sta_plan *p, int32_t *out, int64_t cap, int64_t *count) {
  if (!p || !count) return STA_ERR_ARG;
  *count = (int64_t)p->woff.size();
  if (cap < *count || (!out && *count > 0)) return STA_ERR_ARG;
  if (*count > 0) std::memcpy(out, p->woff.data(), p->woff.size() * sizeof(int32_t));
  return STA_OK;
}

sta_status sta_window_candidates(const int grid[3], int *out, int cap, int *count) {
  if (!grid || !count) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (grid[d] < 1) return STA_ERR_ARG;
  // per axis: the odd extents below the axis length (grid / 2 of them),
  // then the length itself
  int na[3];
  for (int d = 0; d < 3; ++d) na[d] = grid[d] / 2 + 1;
  auto value = [&](int d, int j) { return j < grid[d] / 2 ? 2 * j + 1 : grid[d]; };
  const long long n = (long long)na[0] * na[1] * na[2];
  if (n > INT32_MAX) return STA_ERR_ARG;
  *count = (int)n;
  if (cap < n || !out) return STA_ERR_ARG;
  int i = 0;
  for (int a = 0; a < na[0]; ++a)
    for (int b = 0; b < na[1]; ++b)
      for (int c = 0; c < na[2]; ++c) {
        out[3 * i] = value(0, a); out[3 * i + 1] = value(1, b); out[3 * i + 2] = value(2, c);
        ++i;
      }
  return STA_OK;
}

sta_status sta_window_select(int heads, const int grid[3], const int *candidates, int n_cand,
                             const double *err, double threshold, int *window_out) {
  if (heads < 1 || !grid || !candidates || n_cand < 1 || !err || !window_out) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (grid[d] < 1) return STA_ERR_ARG;
  for (int i = 0; i < 3 * n_cand; ++i)
    if (candidates[i] < 1) return STA_ERR_ARG;
  for (int h = 0; h < heads; ++h) {
    int best = -1;
    long long best_cost = 0;
    double best_err = 0.0;
    for (int c = 0; c < n_cand; ++c) {
      const double e = err[(size_t)h * n_cand + c];
      if (!(e <= threshold)) continue;
      long long cost = 1;
      for (int d = 0; d < 3; ++d) cost *= std::min(candidates[3 * c + d], grid[d]);
      if (best < 0 || cost < best_cost || (cost == best_cost && e < best_err)) {
        best = c; best_cost = cost; best_err = e;
      }
    }
    for (int d = 0; d < 3; ++d) window_out[3 * h + d] = best < 0 ? grid[d] : candidates[3 * best + d];
  }
  return STA_OK;
}

const char *sta_status_string(sta_status s) {
  switch (s) {
    case STA_OK: return "STA_OK";
    case STA_ERR_ARG: return "STA_ERR_ARG: invalid argument";
    case STA_ERR_SHAPE: return "STA_ERR_SHAPE: extent not a multiple of the tile size";
    case STA_ERR_UNSUPPORTED: return "STA_ERR_UNSUPPORTED: unsupported head_dim or tile volume";
    case STA_ERR_ALLOC: return "STA_ERR_ALLOC: allocation failed";
    case STA_ERR_HIP: return "STA_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown sta_status";
}

}  // extern "C"
