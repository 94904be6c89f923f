// Token reorder between natural raster order and tile-major order.
//
// Tiling: the video is cut into non-overlapping tiles ("Fast Video Generation
// with Sliding Tile Attention", gptget summary page, Methodology); in
// tile-major order each tile's tokens are contiguous.  The gather moves whole
// rows of head_dim elements, so it is a pure HBM copy: each thread moves
// 16 bytes, consecutive threads cover consecutive bytes of a row, and a
// wave covers whole rows (256 B rows for bf16, d=128), keeping both the
// reads and the writes coalesced.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sta_launch.h"

namespace sta {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void reorder_kernel(ReorderArgs a) {
  const int cpr = a.row_bytes >> 4;  // 16-byte chunks per row
  const int64_t total = a.rows * cpr;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t row = t / cpr;
    const int chunk = (int)(t - row * cpr);
    const int64_t bh = row / a.N;
    const int p = (int)(row - bh * a.N);      // tile-major position
    const int tile = p / a.V;
    const int nat = a.base[tile] + a.off[p - tile * a.V];
    const int64_t src_row = a.inverse ? row : bh * a.N + nat;
    const int64_t dst_row = a.inverse ? bh * a.N + nat : row;
    const uint4 x = *(reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(a.in) +
                                                      src_row * a.row_bytes) + chunk);
    *(reinterpret_cast<uint4 *>(reinterpret_cast<char *>(a.out) + dst_row * a.row_bytes) + chunk) = x;
  }
}

}  // namespace

hipError_t launch_reorder(const ReorderArgs &a, hipStream_t stream) {
  const int64_t total = a.rows * (a.row_bytes >> 4);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 blocks per compute unit
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sta
