// C-ABI entry points that touch the GPU: device tables, reorder, forward,
// and the process-wide plan cache.  Host-only plan code is in sta_plan.cpp.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "sta_internal.h"
#include "sta_launch.h"

namespace sta {
namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return x < y + nb && y < x + na;
}

// Upload the plan's tables to the current device once; later calls reuse them.
sta_status device_tables(const sta_plan *p, DeviceTables *out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return STA_ERR_HIP;
  std::lock_guard<std::mutex> lock(p->mu);
  auto it = p->dev.find(dev);
  if (it != p->dev.end()) {
    *out = it->second;
    return STA_OK;
  }
  std::vector<int32_t> base_tm(p->n_tiles), off_tm(p->V);
  for (int i = 0; i < p->n_tiles; ++i) base_tm[i] = i * p->V;
  for (int j = 0; j < p->V; ++j) off_tm[j] = j;
  const std::vector<int32_t> *parts[] = {&p->kv_off, &p->kv_idx,   &p->sched,    &p->base_nat,
                                         &p->off_nat, &base_tm,     &off_tm,      &p->q_off,
                                         &p->q_idx,   &p->sched_dq, &p->sched_dkdv, &p->kmask,
                                         &p->swin};
  constexpr int kParts = sizeof(parts) / sizeof(parts[0]);
  size_t offs[kParts], total = 0;
  for (int i = 0; i < kParts; ++i) {
    offs[i] = total;
    total += (parts[i]->size() * sizeof(int32_t) + 255) & ~size_t(255);
  }
  void *block = nullptr;
  if (hipMalloc(&block, total) != hipSuccess) return STA_ERR_ALLOC;
  for (int i = 0; i < kParts; ++i) {
    if (parts[i]->empty()) continue;
    if (hipMemcpy(static_cast<char *>(block) + offs[i], parts[i]->data(),
                  parts[i]->size() * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(block);
      return STA_ERR_HIP;
    }
  }
  DeviceTables t;
  char *b = static_cast<char *>(block);
  t.kv_off = reinterpret_cast<int32_t *>(b + offs[0]);
  t.kv_idx = reinterpret_cast<int32_t *>(b + offs[1]);
  t.sched = reinterpret_cast<int32_t *>(b + offs[2]);
  t.base_nat = reinterpret_cast<int32_t *>(b + offs[3]);
  t.off_nat = reinterpret_cast<int32_t *>(b + offs[4]);
  t.base_tm = reinterpret_cast<int32_t *>(b + offs[5]);
  t.off_tm = reinterpret_cast<int32_t *>(b + offs[6]);
  t.q_off = reinterpret_cast<int32_t *>(b + offs[7]);
  t.q_idx = reinterpret_cast<int32_t *>(b + offs[8]);
  t.sched_dq = reinterpret_cast<int32_t *>(b + offs[9]);
  t.sched_dkdv = reinterpret_cast<int32_t *>(b + offs[10]);
  t.kmask = p->kmask.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[11]);
  t.swin = p->swin.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[12]);
  t.block = block;
  p->dev[dev] = t;
  *out = t;
  return STA_OK;
}

bool valid_dtype(sta_dtype d) { return d == STA_BF16 || d == STA_F32; }
size_t dtype_bytes(sta_dtype d) { return d == STA_F32 ? 4 : 2; }

sta_status reorder(const sta_plan *p, const void *in, void *out, sta_dtype dtype, void *stream,
                   int inverse) {
  if (!p || !in || !out || !valid_dtype(dtype)) return STA_ERR_ARG;
  const size_t bytes = (size_t)p->batch * p->heads * p->N * p->D * dtype_bytes(dtype);
  if (overlaps(in, bytes, out, bytes)) return STA_ERR_ARG;
  if (p->partial || p->swa) return STA_ERR_UNSUPPORTED;   // tile-major order needs whole tiles
  DeviceTables t;
  sta_status st = device_tables(p, &t);
  if (st != STA_OK) return st;
  ReorderArgs a;
  a.in = in;
  a.out = out;
  a.base = t.base_nat;
  a.off = t.off_nat;
  a.rows = (int64_t)p->batch * p->heads * p->N;
  a.N = p->N;
  a.V = p->V;
  a.row_bytes = (int32_t)(p->D * dtype_bytes(dtype));
  a.inverse = inverse;
  return launch_reorder(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STA_OK : STA_ERR_HIP;
}

struct CacheKey {
  std::vector<int> v;
  bool operator<(const CacheKey &o) const { return v < o.v; }
};
std::mutex g_cache_mu;
std::map<CacheKey, sta_plan *> g_cache;

}  // namespace

void release_device_tables(sta_plan *p) {
  std::lock_guard<std::mutex> lock(p->mu);
  if (p->dev.empty()) return;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  // Work launched with the plan may still read its tables: each device
  // finishes its queued work before its copy is freed.
  for (auto &kv : p->dev) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    (void)hipFree(kv.second.block);
  }
  if (have_cur) (void)hipSetDevice(cur);
  p->dev.clear();
}

}  // namespace sta

extern "C" {

sta_status sta_tile_reorder(const sta_plan *plan, const void *in, void *out, sta_dtype dtype,
                            void *stream) {
  return sta::reorder(plan, in, out, dtype, stream, 0);
}

sta_status sta_tile_unreorder(const sta_plan *plan, const void *in, void *out, sta_dtype dtype,
                              void *stream) {
  return sta::reorder(plan, in, out, dtype, stream, 1);
}

}  // extern "C"

namespace sta {
namespace {

sta_status forward(const sta_plan *p, const void *q, const void *k, const void *v, void *out, float *lse,
                   float scale, sta_dtype in_dtype, sta_dtype out_dtype, sta_layout layout, void *stream) {
  if (!p || !q || !k || !v || !out) return STA_ERR_ARG;
  if (!sta::valid_dtype(in_dtype) || !sta::valid_dtype(out_dtype)) return STA_ERR_ARG;
  if (layout != STA_LAYOUT_NATURAL && layout != STA_LAYOUT_TILE_MAJOR) return STA_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return STA_ERR_ARG;
  if ((p->partial || p->swa) && layout != STA_LAYOUT_NATURAL) return STA_ERR_UNSUPPORTED;
  const size_t elems = (size_t)p->batch * p->heads * p->N * p->D;
  const size_t ib = elems * sta::dtype_bytes(in_dtype), ob = elems * sta::dtype_bytes(out_dtype);
  if (sta::overlaps(out, ob, q, ib) || sta::overlaps(out, ob, k, ib) || sta::overlaps(out, ob, v, ib))
    return STA_ERR_ARG;
  if (lse) {
    const size_t lb = (size_t)p->batch * p->heads * p->N * sizeof(float);
    if (overlaps(lse, lb, q, ib) || overlaps(lse, lb, k, ib) || overlaps(lse, lb, v, ib) ||
        overlaps(lse, lb, out, ob))
      return STA_ERR_ARG;
  }
  sta::DeviceTables t;
  sta_status st = sta::device_tables(p, &t);
  if (st != STA_OK) return st;
  sta::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out;
  a.sched = t.sched;
  a.kv_off = t.kv_off;
  a.kv_idx = t.kv_idx;
  a.base = layout == STA_LAYOUT_NATURAL ? t.base_nat : t.base_tm;
  a.off = layout == STA_LAYOUT_NATURAL ? t.off_nat : t.off_tm;
  a.heads = p->heads;
  a.n_tiles = p->n_tiles;
  a.V = p->V;
  a.subs = p->subs;
  a.N = p->N;
  a.sl2e = scale * 1.44269504088896340736f;
  a.n_blocks = (int32_t)p->sched.size();
  a.max_nkv = p->max_nkv;
  a.lse = lse;
  a.kmask = reinterpret_cast<const uint32_t *>(t.kmask);
  a.swin = t.swin;
  a.T = p->T; a.H = p->H; a.W = p->W;
  a.tT = p->tile[0]; a.tH = p->tile[1]; a.tW = p->tile[2];
  a.gH = p->grid[1]; a.gW = p->grid[2];
  hipError_t e = sta::launch_forward(a, p->variant, p->D, in_dtype == STA_F32, out_dtype == STA_F32,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? STA_OK : STA_ERR_HIP;
}

sta_status backward(const sta_plan *p, const void *q, const void *k, const void *v, const void *out,
                    const void *dout, const float *lse, float *delta, void *dq, void *dk, void *dv,
                    float scale, sta_dtype in_dtype, sta_dtype out_dtype, sta_dtype grad_dtype,
                    sta_layout layout, void *stream) {
  if (!p || !q || !k || !v || !out || !dout || !lse || !delta || !dq || !dk || !dv) return STA_ERR_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !valid_dtype(grad_dtype)) return STA_ERR_ARG;
  if (layout != STA_LAYOUT_NATURAL && layout != STA_LAYOUT_TILE_MAJOR) return STA_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return STA_ERR_ARG;
  if (!p->bwd_ok) return STA_ERR_UNSUPPORTED;
  const size_t rows = (size_t)p->batch * p->heads * p->N;
  const size_t elems = rows * p->D;
  const size_t ib = elems * dtype_bytes(in_dtype), ob = elems * dtype_bytes(out_dtype);
  const size_t gb = elems * dtype_bytes(grad_dtype), sb = rows * sizeof(float);
  // Written buffers must not overlap each other or any input.
  const void *written[] = {dq, dk, dv, delta};
  const size_t wbytes[] = {gb, gb, gb, sb};
  const void *read[] = {q, k, v, dout, out, lse};
  const size_t rbytes[] = {ib, ib, ib, ib, ob, sb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(written[i], wbytes[i], read[j], rbytes[j])) return STA_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(written[i], wbytes[i], written[j], wbytes[j])) return STA_ERR_ARG;
  }
  DeviceTables t;
  sta_status st = device_tables(p, &t);
  if (st != STA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_bwd_delta(out, dout, delta, (int64_t)rows, p->D, out_dtype == STA_F32, in_dtype == STA_F32,
                       s) != hipSuccess)
    return STA_ERR_HIP;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.base = layout == STA_LAYOUT_NATURAL ? t.base_nat : t.base_tm;
  a.off = layout == STA_LAYOUT_NATURAL ? t.off_nat : t.off_tm;
  a.heads = p->heads;
  a.n_tiles = p->n_tiles;
  a.V = p->V;
  a.N = p->N;
  a.scale = scale;
  a.sl2e = scale * 1.44269504088896340736f;
  a.f32_out = grad_dtype == STA_F32;
  const bool f32_in = in_dtype == STA_F32;
  a.sched = t.sched_dq;
  a.n_blocks = (int32_t)p->sched_dq.size();
  a.list_off = t.kv_off;
  a.list_idx = t.kv_idx;
  a.max_list = p->max_nkv;
  a.subs = p->bwd_q_subs;
  if (launch_bwd_dq(a, p->bwd_q_waves, p->D, f32_in, s) != hipSuccess) return STA_ERR_HIP;
  a.sched = t.sched_dkdv;
  a.n_blocks = (int32_t)p->sched_dkdv.size();
  a.list_off = t.q_off;
  a.list_idx = t.q_idx;
  a.max_list = p->max_nq;
  a.subs = p->bwd_k_subs;
  if (launch_bwd_dkdv(a, p->bwd_k_pairs, p->D, f32_in, s) != hipSuccess) return STA_ERR_HIP;
  return STA_OK;
}

}  // namespace
}  // namespace sta

extern "C" {

sta_status sta_forward_plan(const sta_plan *p, const void *q, const void *k, const void *v,
                            void *out, float scale, sta_dtype in_dtype, sta_dtype out_dtype,
                            sta_layout layout, void *stream) {
  return sta::forward(p, q, k, v, out, nullptr, scale, in_dtype, out_dtype, layout, stream);
}

sta_status sta_forward_plan_lse(const sta_plan *p, const void *q, const void *k, const void *v,
                                void *out, float *lse, float scale, sta_dtype in_dtype,
                                sta_dtype out_dtype, sta_layout layout, void *stream) {
  if (!lse) return STA_ERR_ARG;
  return sta::forward(p, q, k, v, out, lse, scale, in_dtype, out_dtype, layout, stream);
}

sta_status sta_backward_plan(const sta_plan *p, const void *q, const void *k, const void *v,
                             const void *out, const void *dout, const float *lse, float *delta,
                             void *dq, void *dk, void *dv, float scale, sta_dtype in_dtype,
                             sta_dtype out_dtype, sta_dtype grad_dtype, sta_layout layout,
                             void *stream) {
  return sta::backward(p, q, k, v, out, dout, lse, delta, dq, dk, dv, scale, in_dtype, out_dtype,
                       grad_dtype, layout, stream);
}

sta_status sta_forward(const void *q, const void *k, const void *v, void *out, int batch, int heads,
                       int T, int H, int W, const int tile[3], const int *window, int head_dim,
                       float scale, sta_dtype in_dtype, sta_dtype out_dtype, sta_layout layout,
                       void *stream) {
  if (!tile || !window || heads < 1) return STA_ERR_ARG;
  sta::CacheKey key;
  key.v = {batch, heads, T, H, W, tile[0], tile[1], tile[2], head_dim};
  key.v.insert(key.v.end(), window, window + 3 * heads);
  sta_plan *p = nullptr;
  {
    std::lock_guard<std::mutex> lock(sta::g_cache_mu);
    auto it = sta::g_cache.find(key);
    if (it != sta::g_cache.end()) {
      p = it->second;
    } else {
      sta_status st = sta::build_plan(batch, heads, T, H, W, tile, window, head_dim, false, &p);
      if (st != STA_OK) return st;
      try {
        sta::g_cache[key] = p;
      } catch (...) {
        sta_plan_destroy(p);
        return STA_ERR_ALLOC;
      }
    }
  }
  return sta_forward_plan(p, q, k, v, out, scale, in_dtype, out_dtype, layout, stream);
}

sta_status sta_clear_plan_cache(void) {
  std::lock_guard<std::mutex> lock(sta::g_cache_mu);
  for (auto &kv : sta::g_cache) sta_plan_destroy(kv.second);
  sta::g_cache.clear();
  return STA_OK;
}

}  // extern "C"
