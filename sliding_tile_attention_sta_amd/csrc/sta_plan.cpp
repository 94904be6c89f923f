// Host-side planning for Sliding Tile Attention (no HIP calls in this file).
//
// Geometry follows the STA definition ("Fast Video Generation with Sliding
// Tile Attention", arXiv 2502.04507: index page, Abstract; gptget summary
// page, Methodology and Novelty): non-overlapping 3D tiles, a per-head window
// of whole tiles that slides tile by tile.  Readings where the pages are
// silent: windows wider than the grid are clamped to it, and a window is
// centred on its query tile and shifted inward at the borders.

#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>

#include "sta_internal.h"

namespace sta {
namespace {

inline int window_start(int c, int w, int n) {
  int s = c - (w - 1) / 2;
  if (s < 0) s = 0;
  if (s > n - w) s = n - w;
  return s;
}

// Work items in launch order.  Item code ((b * heads + h) * n_tiles + t) *
// subs + sub; its cost is the length of list (h, t) in off.  Items are
// sorted by decreasing cost, cut into chunks of consecutive items, and each
// chunk goes to the XCD with the least accumulated cost.  Blocks are
// dispatched to XCDs round-robin (block b runs on XCD b % 8), so XCD x's
// queue is placed at blocks x, x + 8, x + 16, ...  Within an XCD the hardware
// hands blocks to free compute units in order, which is list scheduling of a
// decreasing-cost list.  Chunks keep spatially adjacent tiles of one head on
// the same XCD, whose L2 then serves their overlapping windows.
template <typename Off>
std::vector<int32_t> build_schedule(const sta_plan *p, const std::vector<Off> &off, int subs) {
  const int64_t n_items = (int64_t)p->batch * p->heads * p->n_tiles * subs;
  std::vector<int64_t> order(n_items);
  std::iota(order.begin(), order.end(), 0);
  auto cost = [&](int64_t code) {
    int64_t rest = code / subs;
    int t = (int)(rest % p->n_tiles);
    int h = (int)((rest / p->n_tiles) % p->heads);
    return (int64_t)off[(size_t)h * p->n_tiles + t + 1] - off[(size_t)h * p->n_tiles + t];
  };
  std::stable_sort(order.begin(), order.end(),
                   [&](int64_t a, int64_t b) { return cost(a) > cost(b); });

  const int64_t chunk = 32;  // compute units per XCD
  std::vector<std::vector<int32_t>> queue(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (int64_t i = 0; i < n_items; i += chunk) {
    int64_t end = std::min(n_items, i + chunk);
    int64_t c = 0;
    for (int64_t j = i; j < end; ++j) c += cost(order[j]);
    int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += c;
    for (int64_t j = i; j < end; ++j) queue[x].push_back((int32_t)order[j]);
  }
  size_t len = 0;
  for (auto &q : queue) len = std::max(len, q.size());
  std::vector<int32_t> sched(len * kXcds, -1);
  for (int x = 0; x < kXcds; ++x)
    for (size_t s = 0; s < queue[x].size(); ++s) sched[s * kXcds + x] = queue[x][s];
  return sched;
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
    if (fwd_lds_bytes(head_dim, V64, longest) + (partial ? 4LL * longest * (V64 / kKeyBlock) : 0) > kMaxLds)
      return STA_ERR_UNSUPPORTED;
  }

  sta_plan *p = new (std::nothrow) sta_plan();
  if (!p) return STA_ERR_ALLOC;
  try {
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
    if (fwd_lds_bytes(head_dim, p->V, p->max_nkv) + (p->partial ? 4LL * p->max_nkv * (p->V / kKeyBlock) : 0) >
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
#ifndef STA_DKDV_PAIRS
    p->bwd_k_pairs = p->V % 192 == 0 ? 6 : p->V % 128 == 0 ? 4 : 1;
#else
    p->bwd_k_pairs = p->V % (32 * STA_DKDV_PAIRS) == 0 ? STA_DKDV_PAIRS : 1;
#endif
    p->bwd_q_subs = p->V / (32 * p->bwd_q_waves);
    p->bwd_k_subs = p->V / (32 * p->bwd_k_pairs);
    p->bwd_ok = !p->partial && bwd_lds_bytes(head_dim, p->V, std::max(p->max_nkv, p->max_nq)) <= kMaxLds;
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
    p->sched = build_schedule(p, cost_off, p->subs);
  } catch (const std::bad_alloc &) {
    delete p;
    return STA_ERR_ALLOC;
  }
  *out = p;
  return STA_OK;
}

}  // namespace sta

extern "C" {

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
  std::vector<int32_t> list(p->kv_idx.begin() + p->kv_off[i], p->kv_idx.begin() + p->kv_off[i + 1]);
  std::sort(list.begin(), list.end());
  *count = (int)list.size();
  if (!out && cap > 0) return STA_ERR_ARG;
  for (int j = 0; j < cap && j < (int)list.size(); ++j) out[j] = list[j];
  return (int)list.size() > cap ? STA_ERR_ARG : STA_OK;
}

sta_status sta_plan_q_tiles(const sta_plan *p, int head, int kv_tile, int32_t *out, int cap,
                            int *count) {
  if (!p || !count || head < 0 || head >= p->heads || kv_tile < 0 || kv_tile >= p->n_tiles)
    return STA_ERR_ARG;
  const size_t i = (size_t)head * p->n_tiles + kv_tile;
  std::vector<int32_t> list(p->q_idx.begin() + p->q_off[i], p->q_idx.begin() + p->q_off[i + 1]);
  std::sort(list.begin(), list.end());
  const int n = (int)list.size();
  *count = n;
  if (!out && cap > 0) return STA_ERR_ARG;
  for (int j = 0; j < cap && j < n; ++j) out[j] = list[j];
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

sta_status sta_plan_schedule(const sta_plan *p, int32_t *out, int64_t cap, int64_t *count) {
  if (!p || !count) return STA_ERR_ARG;
  *count = (int64_t)p->sched.size();
  if (cap < *count || !out) return STA_ERR_ARG;
  std::memcpy(out, p->sched.data(), p->sched.size() * sizeof(int32_t));
  return STA_OK;
}

sta_status sta_window_candidates(const int grid[3], int *out, int cap, int *count) {
  if (!grid || !count) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (grid[d] < 1) return STA_ERR_ARG;
  std::vector<int> axis[3];
  for (int d = 0; d < 3; ++d) {
    for (int w = 1; w < grid[d]; w += 2) axis[d].push_back(w);
    axis[d].push_back(grid[d]);
  }
  const int n = (int)(axis[0].size() * axis[1].size() * axis[2].size());
  *count = n;
  if (cap < n || !out) return STA_ERR_ARG;
  int i = 0;
  for (int a : axis[0])
    for (int b : axis[1])
      for (int c : axis[2]) {
        out[3 * i] = a; out[3 * i + 1] = b; out[3 * i + 2] = c;
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
