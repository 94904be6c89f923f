// Per-head window search for Sliding Tile Attention.
//
// The pages configure each head's window automatically from the profiled
// locality of its attention ("Fast Video Generation with Sliding Tile
// Attention", arXiv 2502.04507: index page, Abstract; gptget summary page,
// Methodology, Technical Contribution, Novelty and Limitations) without a
// formula.  Reading used here: on calibration inputs, the error of a
// candidate window for head h is ||O_c - O_full|| / ||O_full|| over the
// head's outputs; each head takes the cheapest candidate (fewest key tiles
// per query tile) whose error is within a threshold, else the full window.
//
// The outputs come from the forward kernel (one call per candidate, every
// head at once); the norms from a reduction kernel below, which reads the
// two fp32 outputs once (HBM bound) and writes per-block partial sums that
// the host adds in a fixed order, so the errors are deterministic.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "sta_internal.h"
#include "sta_launch.h"

namespace sta {
namespace {

constexpr int kRedThreads = 256;
constexpr int kRedBlocksPerPlane = 64;

// part[(plane * kRedBlocksPerPlane + blk) * 2 + {0, 1}] =
//   (sum (a - b)^2, sum b^2) over the block's share of one [N, D] plane.
__global__ __launch_bounds__(kRedThreads) void sq_diff_kernel(const float *a, const float *b,
                                                              double *part, int64_t plane_elems) {
  const int64_t plane = blockIdx.y;
  const float4 *pa = reinterpret_cast<const float4 *>(a + plane * plane_elems);
  const float4 *pb = reinterpret_cast<const float4 *>(b + plane * plane_elems);
  const int64_t n4 = plane_elems / 4;
  double sd = 0.0, sr = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; i < n4;
       i += (int64_t)kRedBlocksPerPlane * kRedThreads) {
    const float4 x = pa[i], y = pb[i];
    const float d0 = x.x - y.x, d1 = x.y - y.y, d2 = x.z - y.z, d3 = x.w - y.w;
    sd += (double)(d0 * d0 + d1 * d1) + (double)(d2 * d2 + d3 * d3);
    sr += (double)(y.x * y.x + y.y * y.y) + (double)(y.z * y.z + y.w * y.w);
  }
  __shared__ double red[2][kRedThreads];
  red[0][threadIdx.x] = sd;
  red[1][threadIdx.x] = sr;
  __syncthreads();
  for (int s = kRedThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double *o = part + (plane * kRedBlocksPerPlane + blockIdx.x) * 2;
    o[0] = red[0][0];
    o[1] = red[1][0];
  }
}

struct DevBuf {
  void *p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

struct PlanHolder {
  sta_plan *p = nullptr;
  ~PlanHolder() {
    if (p) sta_plan_destroy(p);
  }
};

}  // namespace
}  // namespace sta

extern "C" {

sta_status sta_window_errors(const void *q, const void *k, const void *v, int batch, int heads, int T,
                             int H, int W, const int tile[3], int head_dim, float scale,
                             sta_dtype in_dtype, sta_layout layout, const int *candidates,
                             int n_cand, double *err, void *stream) {
  if (!q || !k || !v || !tile || !candidates || !err || n_cand < 1 || heads < 1 || batch < 1)
    return STA_ERR_ARG;
  for (int i = 0; i < 3 * n_cand; ++i)
    if (candidates[i] < 1) return STA_ERR_ARG;
  for (int d = 0; d < 3; ++d)
    if (tile[d] < 1) return STA_ERR_ARG;
  const int ext[3] = {T, H, W};
  for (int d = 0; d < 3; ++d)
    if (ext[d] < 1) return STA_ERR_ARG;
  // Extents that are not multiples of the tile: plans with partial tiles
  // (ceil(extent / tile) tiles per axis, only existing tokens take part).
  bool partial = false;
  for (int d = 0; d < 3; ++d) partial |= ext[d] % tile[d] != 0;
  const int flags = partial ? STA_PLAN_PARTIAL_TILES : 0;
  if (partial && layout != STA_LAYOUT_NATURAL) return STA_ERR_UNSUPPORTED;   // tile-major needs whole tiles
  const int grid[3] = {(T + tile[0] - 1) / tile[0], (H + tile[1] - 1) / tile[1], (W + tile[2] - 1) / tile[2]};
  const int64_t plane = (int64_t)T * H * W * head_dim;
  const size_t out_bytes = (size_t)batch * heads * plane * sizeof(float);
  const size_t part_count = (size_t)batch * heads * sta::kRedBlocksPerPlane * 2;
  // Host buffers first: nothing below allocates on the host once work is
  // queued (the entry point never throws).
  std::vector<int> win;
  std::vector<double> host;
  try {
    win.resize((size_t)heads * 3);
    host.resize(part_count);
  } catch (const std::bad_alloc &) {
    return STA_ERR_ALLOC;
  }

  // Full-attention plan (window = grid for every head) and its output.
  for (int h = 0; h < heads; ++h)
    for (int d = 0; d < 3; ++d) win[h * 3 + d] = grid[d];
  sta::PlanHolder full;
  sta_status st = sta_plan_create_ex(batch, heads, T, H, W, tile, win.data(), head_dim, flags, &full.p);
  if (st != STA_OK) return st;
  int dev = -1;   // (after the argument checks, before any allocation on a device)
  if (hipGetDevice(&dev) != hipSuccess) return STA_ERR_HIP;
  sta::DevBuf ref, cand, part;
  if (sta::test_fail_alloc() || hipMalloc(&ref.p, out_bytes) != hipSuccess || hipMalloc(&cand.p, out_bytes) != hipSuccess ||
      hipMalloc(&part.p, part_count * sizeof(double)) != hipSuccess)
    return STA_ERR_ALLOC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Once work is queued, every exit drains the stream before the plans and
  // buffers it uses are released.
  auto fail = [&](sta_status e) {
    (void)hipStreamSynchronize(s);
    return e;
  };
  st = sta_forward_plan(full.p, q, k, v, ref.p, scale, in_dtype, STA_F32, layout, stream);
  if (st != STA_OK) return fail(st);

  // Candidate c's plan is built on the host while the GPU runs candidate
  // c - 1 (two plans alive at a time); a plan goes once the stream has
  // drained after its launches.
  sta::PlanHolder cp[2];
  auto make = [&](int c, sta::PlanHolder &h) {
    for (int hh = 0; hh < heads; ++hh)
      for (int d = 0; d < 3; ++d) win[hh * 3 + d] = candidates[c * 3 + d];
    return sta_plan_create_ex(batch, heads, T, H, W, tile, win.data(), head_dim, flags, &h.p);
  };
  st = make(0, cp[0]);
  if (st != STA_OK) return fail(st);
  for (int c = 0; c < n_cand; ++c) {
    sta::PlanHolder &cur = cp[c & 1], &nxt = cp[(c + 1) & 1];
    st = sta_forward_plan(cur.p, q, k, v, cand.p, scale, in_dtype, STA_F32, layout, stream);
    if (st != STA_OK) return fail(st);
    hipLaunchKernelGGL(sta::sq_diff_kernel, dim3(sta::kRedBlocksPerPlane, batch * heads),
                       dim3(sta::kRedThreads), 0, s, static_cast<const float *>(cand.p),
                       static_cast<const float *>(ref.p), static_cast<double *>(part.p), plane);
    if (hipGetLastError() != hipSuccess) return fail(STA_ERR_HIP);
    // (before the copy: a copy into pageable host memory may block the host)
    if (c + 1 < n_cand) {
      st = make(c + 1, nxt);
      if (st != STA_OK) return fail(st);
    }
    if (hipMemcpyAsync(host.data(), part.p, part_count * sizeof(double), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(STA_ERR_HIP);
    sta_plan_destroy(cur.p);
    cur.p = nullptr;
    for (int h = 0; h < heads; ++h) {
      double sd = 0.0, sr = 0.0;
      for (int b = 0; b < batch; ++b)
        for (int i = 0; i < sta::kRedBlocksPerPlane; ++i) {
          const double *x = &host[(((size_t)b * heads + h) * sta::kRedBlocksPerPlane + i) * 2];
          sd += x[0];
          sr += x[1];
        }
      err[(size_t)h * n_cand + c] = sr > 0.0 ? std::sqrt(sd) / std::sqrt(sr) : (sd > 0.0 ? INFINITY : 0.0);
    }
  }
  return STA_OK;
}

sta_status sta_window_search(const void *const *q, const void *const *k, const void *const *v,
                             int n_samples, int batch, int heads, int T, int H, int W, const int tile[3],
                             int head_dim, float scale, sta_dtype in_dtype, sta_layout layout,
                             const int *candidates, int n_cand, double threshold, double *err_out,
                             int *window_out, void *stream) {
  if (!q || !k || !v || n_samples < 1 || !tile || !candidates || n_cand < 1 || heads < 1 || !window_out)
    return STA_ERR_ARG;
  for (int i = 0; i < n_samples; ++i)
    if (!q[i] || !k[i] || !v[i]) return STA_ERR_ARG;
  std::vector<double> one, mean;
  try {
    one.resize((size_t)heads * n_cand);
    mean.assign((size_t)heads * n_cand, 0.0);
  } catch (const std::bad_alloc &) {
    return STA_ERR_ALLOC;
  }
  // W1, W2 per sample; W4: the arithmetic mean over the samples, summed in
  // sample order
  for (int i = 0; i < n_samples; ++i) {
    const sta_status st = sta_window_errors(q[i], k[i], v[i], batch, heads, T, H, W, tile, head_dim, scale,
                                            in_dtype, layout, candidates, n_cand, one.data(), stream);
    if (st != STA_OK) return st;
    for (size_t j = 0; j < one.size(); ++j) mean[j] += one[j];
  }
  for (double &x : mean) x /= n_samples;
  if (err_out)
    for (size_t j = 0; j < mean.size(); ++j) err_out[j] = mean[j];
  // W3 on the mean, over the grid of (possibly partial) tiles
  const int grid[3] = {(T + tile[0] - 1) / tile[0], (H + tile[1] - 1) / tile[1], (W + tile[2] - 1) / tile[2]};
  return sta_window_select(heads, grid, candidates, n_cand, mean.data(), threshold, window_out);
}

}  // extern "C"
