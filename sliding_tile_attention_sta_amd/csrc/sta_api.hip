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

// Orders `stream` after the upload of the tables in t (a no-op on the
// stream that uploaded them).
sta_status wait_upload(const DeviceTables &t, void *stream) {
  if (t.ready == nullptr || t.upload_stream == stream) return STA_OK;
  return hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(t.ready), 0) == hipSuccess
             ? STA_OK
             : STA_ERR_HIP;
}

// Upload the plan's tables to the current device once, with asynchronous
// copies on the caller's stream (the host sources live as long as the plan);
// later calls reuse them.
sta_status device_tables(const sta_plan *p, void *stream, DeviceTables *out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return STA_ERR_HIP;
  std::lock_guard<std::mutex> lock(p->mu);
  auto it = p->dev.find(dev);
  if (it != p->dev.end()) {
    *out = it->second;
    return wait_upload(it->second, stream);
  }
  const std::vector<int32_t> *parts[] = {&p->kv_off, &p->kv_idx,   &p->sched,    &p->base_nat,
                                         &p->off_nat, &p->base_tm,  &p->off_tm,   &p->q_off,
                                         &p->q_idx,   &p->sched_dq, &p->sched_dkdv, &p->kmask,
                                         &p->swin,    &p->ptab,     &p->gtab,     &p->queue,
                                         &p->wlist,   &p->woff};
  constexpr int kParts = sizeof(parts) / sizeof(parts[0]);
  size_t offs[kParts], total = 0;
  for (int i = 0; i < kParts; ++i) {
    offs[i] = total;
    total += (parts[i]->size() * sizeof(int32_t) + 255) & ~size_t(255);
  }
  void *block = nullptr;
  if (test_fail_alloc() || hipMalloc(&block, total) != hipSuccess) return STA_ERR_ALLOC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ready = nullptr;
  auto fail = [&](sta_status e) {
    (void)hipStreamSynchronize(s);
    if (ready) (void)hipEventDestroy(ready);
    (void)hipFree(block);
    return e;
  };
  for (int i = 0; i < kParts; ++i) {
    if (parts[i]->empty()) continue;
    if (hipMemcpyAsync(static_cast<char *>(block) + offs[i], parts[i]->data(),
                       parts[i]->size() * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess)
      return fail(STA_ERR_HIP);
  }
  if (hipEventCreateWithFlags(&ready, hipEventDisableTiming) != hipSuccess) {
    ready = nullptr;
    return fail(STA_ERR_HIP);
  }
  if (hipEventRecord(ready, s) != hipSuccess) return fail(STA_ERR_HIP);
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
  t.ptab = p->ptab.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[13]);
  t.gtab = p->gtab.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[14]);
  t.queue = p->queue.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[15]);
  t.wlist = p->woff.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[16]);
  t.woff = p->woff.empty() ? nullptr : reinterpret_cast<int32_t *>(b + offs[17]);
  t.block = block;
  t.upload_stream = stream;
  t.ready = ready;
  try {
    p->dev[dev] = t;
  } catch (const std::bad_alloc &) {
    return fail(STA_ERR_ALLOC);
  }
  *out = t;
  return STA_OK;
}

// The plan's tables on the current device if they were uploaded before
// (no allocation); STA_ERR_UNSUPPORTED if not.
sta_status existing_device_tables(const sta_plan *p, void *stream, DeviceTables *out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return STA_ERR_HIP;
  std::lock_guard<std::mutex> lock(p->mu);
  auto it = p->dev.find(dev);
  if (it == p->dev.end()) return STA_ERR_UNSUPPORTED;
  *out = it->second;
  return wait_upload(it->second, stream);
}

// Scratch of sta_forward_plan_noalloc: a fixed array in device memory that
// each device holds while the library is loaded, shared by every such call
// on that device.  64 MiB: the queue words and arrival counters of any plan
// and the partial-result slots of up to about 320 pieces at head_dim 128
// (the 720p and 60x48x80 workloads use 256).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) int32_t scratch[kStaticScratchBytes / 4];
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void *g_static_ptr[kMaxDevices] = {};   // device address of scratch, per device

// The device address of scratch on the current device.  Looked up once per
// device (hipGetSymbolAddress, with that device current); in host code the
// array's name is only a stand-in, never a device address.
sta_status static_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return STA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return STA_ERR_HIP;
    g_static_ptr[dev] = ptr;
  }
  *out = g_static_ptr[dev];
  return STA_OK;
}

// Debug builds: one word per device that the kernels' bounds checks set
// bits in (see STA_CHECK), at a device address looked up once per device.
#ifdef STA_DEBUG
static __device__ unsigned dbg_word;
unsigned *g_dbg_ptr[kMaxDevices] = {};
unsigned *debug_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_dbg_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(dbg_word)) != hipSuccess) return nullptr;
    g_dbg_ptr[dev] = static_cast<unsigned *>(ptr);
  }
  return g_dbg_ptr[dev];
}
#else
unsigned *debug_word() { return nullptr; }
#endif

// The forward scratch of a plan with dynamic queues on the current device,
// for launches on `stream` (allocated on first use; its counters are
// cleared once, in stream order, and every launch leaves them zero).
sta_status forward_scratch(const sta_plan *p, void *stream, void **out) {
  *out = nullptr;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return STA_ERR_HIP;
  std::lock_guard<std::mutex> lock(p->mu);
  const auto key = std::make_pair(dev, stream);
  auto it = p->scratch.find(key);
  if (it != p->scratch.end()) {
    *out = it->second;
    return STA_OK;
  }
  void *buf = nullptr;
  if (test_fail_alloc() || hipMalloc(&buf, (size_t)p->fwd_scratch()) != hipSuccess)
    return STA_ERR_ALLOC;
  if (launch_zero(static_cast<int32_t *>(buf), (int)fwd_zero_words(p->n_groups, p->items()),
                  static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipFree(buf);
    return STA_ERR_HIP;
  }
  try {
    p->scratch[key] = buf;
  } catch (...) {
    (void)hipFree(buf);
    return STA_ERR_ALLOC;
  }
  *out = buf;
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
  sta_status st = device_tables(p, stream, &t);
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

}  // namespace

void release_device_tables(sta_plan *p) {
  std::lock_guard<std::mutex> lock(p->mu);
  if (p->dev.empty() && p->scratch.empty()) return;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  // Work launched with the plan may still read its tables and scratch: each
  // device finishes its queued work before its buffers are freed.  (No
  // allocation here: destroying a plan cannot fail.)
  bool synced[kMaxDevices] = {};
  auto sync = [&](int dev) {
    if (dev >= 0 && dev < kMaxDevices && synced[dev]) return true;
    if (hipSetDevice(dev) != hipSuccess) return false;
    (void)hipDeviceSynchronize();
    if (dev >= 0 && dev < kMaxDevices) synced[dev] = true;
    return true;
  };
  for (auto &kv : p->dev)
    if (sync(kv.first)) {
      if (kv.second.ready) (void)hipEventDestroy(static_cast<hipEvent_t>(kv.second.ready));
      (void)hipFree(kv.second.block);
    }
  for (auto &kv : p->scratch)
    if (sync(kv.first.first)) (void)hipFree(kv.second);
  if (have_cur) (void)hipSetDevice(cur);
  p->dev.clear();
  p->scratch.clear();
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

// no_alloc: use the plan's device tables only if they exist, and the
// library's static scratch (cleared by a kernel at every call) instead of a
// per-stream allocation.
sta_status forward(const sta_plan *p, const void *q, const void *k, const void *v, void *out, float *lse,
                   float scale, sta_dtype in_dtype, sta_dtype out_dtype, sta_layout layout, void *stream,
                   bool no_alloc = false) {
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
  void *scratch = nullptr;
  if (no_alloc) {
    if (p->fwd_scratch() > (long long)kStaticScratchBytes) return STA_ERR_UNSUPPORTED;
    sta_status st = existing_device_tables(p, stream, &t);
    if (st != STA_OK) return st;
    st = static_scratch(&scratch);
    if (st != STA_OK) return st;
    if (launch_zero(static_cast<int32_t *>(scratch), (int)fwd_zero_words(p->n_groups, p->items()),
                    static_cast<hipStream_t>(stream)) != hipSuccess)
      return STA_ERR_HIP;
  } else {
    sta_status st = sta::device_tables(p, stream, &t);
    if (st != STA_OK) return st;
    st = forward_scratch(p, stream, &scratch);
    if (st != STA_OK) return st;
  }
  sta::FwdArgs a{};
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
  // Per-step addressing of K and V: blocks that are a first row plus
  // per-position offsets, a step table that fits in LDS beside the stages
  // (and the validity words of partial tiles), and byte offsets below 2 GiB
  // for every row a tile position names in one (batch, head): partial
  // tiles name rows past the tensor, which the buffer loads' range check
  // reads as zeros.
  const long long last_row = p->partial ? (long long)p->base_nat.back() + p->off_nat.back() : p->N - 1;
  a.sep = !p->swa && (layout == STA_LAYOUT_TILE_MAJOR || p->sep_nat) &&
          fwd_lds_bytes(p->D, p->V, p->max_nkv) +
                  (p->partial ? 2 : 1) * fwd_lds_step_bytes(p->V, p->max_nkv) <= kMaxLds &&
          std::max<long long>(last_row + 1, p->N) * p->D * (long long)dtype_bytes(in_dtype) < (1LL << 31);
  a.kmask = reinterpret_cast<const uint32_t *>(t.kmask);
  a.swin = t.swin;
  a.T = p->T; a.H = p->H; a.W = p->W;
  a.tT = p->tile[0]; a.tH = p->tile[1]; a.tW = p->tile[2];
  a.gH = p->grid[1]; a.gW = p->grid[2];
  a.queue = t.queue;
  for (int x = 0; x < 10; ++x) a.qoff[x] = p->qoff[x];
  a.qcount = static_cast<int32_t *>(scratch);
  if (p->dyn_blocks) a.n_blocks = p->dyn_blocks;
  a.ptab = t.ptab;
  a.gtab = t.gtab;
  a.wlist = t.wlist;
  a.woff = t.woff;
  if (!p->woff.empty()) a.n_blocks = (int32_t)p->woff.size() - 1;
  a.pcount = a.qcount + kQueueWords;
  a.fbits = reinterpret_cast<unsigned *>(a.pcount + p->n_groups);
  a.flist = a.qcount + fwd_zero_words(p->n_groups, p->items());
  a.pslot = p->n_pieces ? reinterpret_cast<float *>(static_cast<char *>(scratch) +
                                                    fwd_counter_bytes(p->n_groups, p->items()))
                        : nullptr;
  a.n_items = (int32_t)p->items();
  a.n_pieces = p->n_pieces;
  a.dbg = debug_word();
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
  if (p->partial && layout != STA_LAYOUT_NATURAL) return STA_ERR_UNSUPPORTED;   // tile-major needs whole tiles
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
  sta_status st = device_tables(p, stream, &t);
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
  a.kmask = reinterpret_cast<const uint32_t *>(t.kmask);
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
  a.n_items = p->batch * p->heads * p->n_tiles * p->bwd_q_subs;
  a.dbg = debug_word();
  if (launch_bwd_dq(a, p->bwd_q_waves, p->D, f32_in, s) != hipSuccess) return STA_ERR_HIP;
  a.sched = t.sched_dkdv;
  a.n_blocks = (int32_t)p->sched_dkdv.size();
  a.list_off = t.q_off;
  a.list_idx = t.q_idx;
  a.max_list = p->max_nq;
  a.subs = p->bwd_k_subs;
  a.n_items = p->batch * p->heads * p->n_tiles * p->bwd_k_subs;
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

sta_status sta_forward_plan_noalloc(const sta_plan *p, const void *q, const void *k, const void *v,
                                    void *out, float *lse, float scale, sta_dtype in_dtype,
                                    sta_dtype out_dtype, sta_layout layout, void *stream) {
  return sta::forward(p, q, k, v, out, lse, scale, in_dtype, out_dtype, layout, stream, true);
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
  sta_status st = STA_OK;
  const std::shared_ptr<sta_plan> p = sta::cached_plan(batch, heads, T, H, W, tile, window, head_dim, &st);
  if (!p) return st;
  return sta_forward_plan(p.get(), q, k, v, out, scale, in_dtype, out_dtype, layout, stream);
}

sta_status sta_debug_flags(uint32_t *flags, int clear) {
  if (!flags) return STA_ERR_ARG;
  *flags = 0;
#ifdef STA_DEBUG
  unsigned *w = sta::debug_word();
  if (!w) return STA_ERR_HIP;
  if (hipMemcpy(flags, w, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess) return STA_ERR_HIP;
  if (clear) {
    const unsigned zero = 0;
    if (hipMemcpy(w, &zero, sizeof(unsigned), hipMemcpyHostToDevice) != hipSuccess) return STA_ERR_HIP;
  }
  return STA_OK;
#else
  (void)clear;
  return STA_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
