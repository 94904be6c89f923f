// Sliding Tile Attention forward for gfx950 (MI355X).
//
// What is computed ("Fast Video Generation with Sliding Tile Attention",
// arXiv 2502.04507, index page, Abstract; gptget summary page, Methodology and
// Novelty): every query tile attends to the whole key/value tiles of its 3D
// window and to nothing else.  Because a (query tile, key tile) pair is
// either fully attended or skipped, the kernel never evaluates a mask: it
// walks the key-tile list of its query tile and runs dense blocks.  The
// summary page credits the original kernel's speed to dense computation on
// the sparse pattern in the FlashAttention line (softmax over streamed key
// blocks); this kernel keeps that idea and is otherwise laid out for CDNA4:
//
//   * One work group owns QPI query tokens of one (batch, head, query tile)
//     and keeps them for the whole window; each wave owns 16*QB queries.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_bf16: K comes from LDS, Q stays in VGPRs.  In the
//     accumulator layout a lane holds one query and 4 keys of each 16x16
//     block.
//   * Softmax in fp32 with exp2 and the scale folded into one FMA, against
//     one reference max per query row that starts as the row's max over the
//     first key block and moves only when it must: probabilities are rounded
//     to fp16 (nearest even), which holds values up to 65504, so a block
//     whose scores exceed the reference by less than 16 (exp2 units) needs
//     nothing, and a larger excess overflows to +inf in the row sum, which a
//     compare per step detects and a rare repair fixes (new reference = row
//     max, O and l rescaled, the block's probabilities recomputed).  A step
//     therefore computes no row max, which takes about a third of the VALU
//     work off it (the kernel is bound by VALU issue more than by the MFMAs).
//   * fp16 keeps 11 significant bits against bf16's 8, which cuts the error
//     of the weighted sum about tenfold when a few keys dominate a row.  The
//     row sum is accumulated from the rounded probabilities with
//     v_dot2_f32_f16, so numerator and denominator use the same values.
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_f16.  V is converted to fp16 as
//     it is staged into LDS.  The V^T operand is read from row-major V in LDS
//     with ds_read_b64_tr_b16, which transposes 4x16 16-bit blocks inside
//     each 16-lane group, so V is never transposed in memory.
//   * K and V advance 32 keys at a time through two-stage LDS rings; the
//     next blocks' global loads are issued before the current block's math.
//   * The two waves sharing a SIMD run each step in opposite orders
//     (ping-pong), so one wave's softmax VALU work overlaps the other's MFMAs.
//   * Rows are located through two small tables (tile base row, tile-local
//     row offset), so one kernel reads and writes either the natural
//     [T, H, W] token order or the tile-major order.
//   * Partial tiles (an extent that is not a multiple of its tile size; a
//     separate instantiation, PARTIAL): rows are clamped to the tensor (with
//     per-step addressing, rows past it read as zeros instead), the
//     scores of keys that do not exist are set to -inf from a per-tile
//     validity bitmask (one 32-bit word per 32-key block), and queries that
//     do not exist are not stored.  Only tiles at the video's far edges
//     hold such tokens.
//   * Token-wise sliding window attention (SWA, a separate instantiation):
//     the baseline STA is contrasted with, for measurement.  Each query has
//     its own window of tokens centred on itself (shifted inward at the
//     borders); a query tile walks the union of its queries' windows in
//     runs of 32 keys along W, and every score is masked against its
//     query's window.  The row's reference max starts at the query's score
//     against its own key, which every window holds (the first key block
//     may hold none of a query's keys).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"
#include "sta_launch.h"

namespace sta {
namespace {

constexpr int KB = kKeyBlock;  // keys per pipeline step

// Max / sum of x over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float swap_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float swap_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Token-wise SWA: first token of the w-token window of coordinate x on an
// axis of extent e (w <= e).
__device__ __forceinline__ int tok_start(int x, int w, int e) {
  const int s = x - (w - 1) / 2;
  return s < 0 ? 0 : (s > e - w ? e - w : s);
}

// D: head dim.  QB: 16-query blocks per wave.  NW: waves per group.
template <int D, int QB, int NW, bool F32IN, bool F32OUT, bool PARTIAL, bool SWA = false, bool SEP = false,
          bool FIXUP = false, bool MULTI = false>
__global__ __launch_bounds__(NW * 64) void sta_fwd_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int QPI = 16 * QB * NW;               // queries per work item
  constexpr int KSTR = fwd_kstride(D);            // padded LDS row strides (bytes)
  constexpr int VSTR = fwd_vstride(D);
  constexpr int KST_BYTES = KB * KSTR;
  constexpr int VST_BYTES = KB * VSTR;
  constexpr int CHUNKS = KB * D / 8;              // 8-element chunks per tensor per step
  constexpr int CPT = (CHUNKS + NT - 1) / NT;     // chunks per thread per tensor
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "chunk split");
  constexpr int EB = F32IN ? 4 : 2;               // input element bytes
  constexpr int DC = D / 32;                      // 32-wide d chunks (QK^T K-dim steps)
  constexpr int DB = D / 16;                      // 16-wide d blocks (rows of O^T)

  // LDS: K stages, V stages, tile-local row offsets, key-tile base rows.
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int *off_l = reinterpret_cast<int *>(smem + 2 * KST_BYTES + 2 * VST_BYTES);
  int *kvb_l = off_l + a.V;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // The work item.  Dynamic queues: thread 0 takes the next entry of its
  // XCD's queue (hardware register XCC_ID), or of the next XCD queue that
  // is not empty, or else of the piece queue, and shares it through LDS; a
  // work group that finds every queue empty exits (and sets a flag that
  // lets later ones exit at once).  Every work group counts itself out at
  // its end, and the last one zeroes the queue words for the next launch.
  // The item is uniform: readfirstlane keeps it and everything derived from
  // it in SGPRs.  A piece of a split item walks steps [s_first, s_end) of
  // the item's key blocks.
  __shared__ int last_piece;      // a split item's piece: the last one to arrive
  __shared__ unsigned vmax_bits;  // FIXUP: largest |v| of the item's keys
  int item = -1;
  if constexpr (FIXUP || MULTI) {
  } else if (a.queue != nullptr) {
    __shared__ int taken;
    if (tid == 0) {
      int code = -1;
      const int x = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7);   // HW_REG_XCC_ID[3:0]
      for (int t = 0; t < 9; ++t) {
        const int y = t == 8 ? 8 : (x + t) & 7;
        const int n = a.qoff[y + 1] - a.qoff[y];
        if (n == 0) continue;
        if (t == 1 && __hip_atomic_load(a.qcount + 10, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        const int i = atomicAdd(a.qcount + y, 1);
        if (i < n) {
          code = a.queue[a.qoff[y] + i];
          break;
        }
      }
      if (code == -1) __hip_atomic_store(a.qcount + 10, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      taken = code;
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(taken);
  } else {
    item = __builtin_amdgcn_readfirstlane(a.sched[blockIdx.x]);
  }
  auto finish = [&]() {
    if (a.queue != nullptr && tid == 0 && atomicAdd(a.qcount + 9, 1) == a.n_blocks - 1) {
      // queue counters, finished work groups, empty flag (the marked items'
      // count is the fix-up kernel's to read and reset)
      for (int i = 0; i < 11; ++i) __hip_atomic_store(a.qcount + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (!FIXUP && !MULTI && item == -1) {
    finish();
    return;
  }
  // MULTI (plans with fewer work items than compute units): work group b
  // runs the entries wlist[woff[b] .. woff[b+1]) in turn, whole items and
  // pieces of one contiguous range of the launch's key steps, so that every
  // compute unit walks the same number of steps.
  int w_k = 0, w_end = 0;
  if constexpr (MULTI) {
    w_k = __builtin_amdgcn_readfirstlane(a.woff[blockIdx.x]);
    w_end = __builtin_amdgcn_readfirstlane(a.woff[blockIdx.x + 1]);
  }
  // FIXUP: the items the forward marked (V beyond fp16's range, see the
  // check after the walk), taken in turn by the work groups and redone with
  // V scaled; the last work group out clears the marks for the next launch.
  int nbad = 0, fix_k = blockIdx.x;
  if constexpr (FIXUP) {
    nbad = __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.qcount + 11, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT));
    if (nbad == 0) return;
  }
next_item:
  if constexpr (FIXUP) {
    if (fix_k >= nbad) {
      if (tid == 0 && atomicAdd(a.qcount + 12, 1) == (int)gridDim.x - 1) {
        for (int k = 0; k < nbad; ++k)
          __hip_atomic_store(a.fbits + (a.flist[k] >> 5), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.qcount + 11, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.qcount + 12, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    item = __builtin_amdgcn_readfirstlane(a.flist[fix_k]);
    fix_k += gridDim.x;
  } else if constexpr (MULTI) {
    if (w_k >= w_end) return;
    item = __builtin_amdgcn_readfirstlane(a.wlist[w_k]);
    ++w_k;
  }
  int piece = -1, s_first = 0, s_end = 0;
  if (item < -1) {
    piece = -2 - item;
    STA_CHECK(a.dbg, piece < a.n_pieces, 0);
    item = __builtin_amdgcn_readfirstlane(a.ptab[4 * piece]);
    s_first = __builtin_amdgcn_readfirstlane(a.ptab[4 * piece + 1]);
    s_end = __builtin_amdgcn_readfirstlane(a.ptab[4 * piece + 2]);
  }
  STA_CHECK(a.dbg, item >= 0 && item < a.n_items, 0);
  const int sub = item % a.subs;
  const int rest = item / a.subs;
  const int qt = rest % a.n_tiles;
  const int bh = rest / a.n_tiles;
  const int h = bh % a.heads;

  // Work-item constants are wave-uniform; readfirstlane keeps them in SGPRs
  // so that the key loop is a scalar (non-divergent) loop.
  int kv0 = 0, nkv = 0;
  if constexpr (!SWA) {
    kv0 = __builtin_amdgcn_readfirstlane(a.kv_off[h * a.n_tiles + qt]);
    nkv = __builtin_amdgcn_readfirstlane(a.kv_off[h * a.n_tiles + qt + 1]) - kv0;
  }
  for (int i = tid; i < a.V; i += NT) off_l[i] = a.off[i];
  for (int i = tid; i < nkv; i += NT) {
    STA_CHECK(a.dbg, (unsigned)a.kv_idx[kv0 + i] < (unsigned)a.n_tiles && i < a.max_nkv, 1);
    kvb_l[i] = a.base[a.kv_idx[kv0 + i]];
  }
  // SWA: the union box of the tile's query windows, walked as rows (t, y)
  // of nzb runs of 32 keys starting at z = z_lo.
  int s_wt = 0, s_wy = 0, s_wz = 0, s_tlo = 0, s_ylo = 0, s_zlo = 0, s_ny = 1, s_nzb = 1, s_nrows = 0;
  if constexpr (SWA) {
    s_wt = a.swin[3 * h]; s_wy = a.swin[3 * h + 1]; s_wz = a.swin[3 * h + 2];
    const int ct = qt / (a.gH * a.gW), cy = (qt / a.gW) % a.gH, cz = qt % a.gW;
    s_tlo = tok_start(ct * a.tT, s_wt, a.T);
    s_ylo = tok_start(cy * a.tH, s_wy, a.H);
    s_zlo = tok_start(cz * a.tW, s_wz, a.W);
    const int thi = tok_start(ct * a.tT + a.tT - 1, s_wt, a.T) + s_wt;
    const int yhi = tok_start(cy * a.tH + a.tH - 1, s_wy, a.H) + s_wy;
    const int zhi = tok_start(cz * a.tW + a.tW - 1, s_wz, a.W) + s_wz;
    s_ny = yhi - s_ylo;
    s_nzb = (zhi - s_zlo + KB - 1) / KB;
    s_nrows = (thi - s_tlo) * s_ny;
  }
  // PARTIAL: the validity word of every 32-key block of the walk.
  uint32_t *mw_l = reinterpret_cast<uint32_t *>(kvb_l + a.max_nkv);
  if constexpr (PARTIAL) {
    const int words = a.V / KB;
    for (int i = tid; i < nkv * words; i += NT)
      mw_l[i] = a.kmask[(size_t)a.kv_idx[kv0 + i / words] * words + i % words];
  }
  // SEP: the byte offset of the first key row of every 32-key block of the
  // walk (the rows of a block are that row plus a fixed offset per position),
  // after the validity words when both are used.
  int *stp_l = reinterpret_cast<int *>(kvb_l + a.max_nkv) + (PARTIAL ? a.max_nkv * (a.V / KB) : 0);
  if constexpr (SEP) {
    const int spb = a.V / KB;
    for (int i = tid; i < nkv * spb; i += NT)
      stp_l[i] = (a.base[a.kv_idx[kv0 + i / spb]] + a.off[(i % spb) * KB]) * (D * EB);
  }

  const char *qg = reinterpret_cast<const char *>(a.q) + (size_t)bh * a.N * D * EB;
  const char *kg = reinterpret_cast<const char *>(a.k) + (size_t)bh * a.N * D * EB;
  const char *vg = reinterpret_cast<const char *>(a.v) + (size_t)bh * a.N * D * EB;
  const int qbase = a.base[qt];
  const int qloc0 = sub * QPI + wave * 16 * QB;
  __syncthreads();

  // ---- Q fragments (B operand of S^T = K Q^T), kept in VGPRs --------------
  bf16x8 qf[QB][DC];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    int row = qbase + off_l[qloc0 + 16 * j + l16];
    if constexpr (PARTIAL) row = row < a.N ? row : (int)a.N - 1;
    STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N && qloc0 + 16 * j + l16 < a.V, 2);
#pragma unroll
    for (int c = 0; c < DC; ++c)
      qf[j][c] = __builtin_bit_cast(bf16x8, as_bf16<F32IN>(load_raw<F32IN>(
                                              qg + ((size_t)row * D + 32 * c + 8 * g) * EB)));
  }

  // ---- key-tile walk ------------------------------------------------------
  const int spt = SWA ? s_nzb : a.V / KB;   // steps per key tile (SWA: per key row)
  if (piece < 0) s_end = SWA ? s_nrows * s_nzb : nkv * spt;
  const int nsteps = s_end - s_first;      // steps of this work group

  // Global -> register prefetch of one 32-key block of K and of V.  The rows
  // of the next fetch are looked up (LDS tables) right after the current one
  // is issued, so the lookups never delay a step's global loads.
  Raw8<F32IN> rk[CPT], rv[CPT];
  // key tile / step-in-tile of the next fetch
  int fk_ti = s_first / spt, fk_u = s_first % spt, fv_ti = fk_ti, fv_u = fk_u;
  int krow[CPT], vrow[CPT];                        // token rows of the next fetch
  auto rows_at = [&](int (&nrow)[CPT], int ti, int u) {
    if constexpr (SWA) {
      // ti = key row (t, y) of the union box, u = 32-key run along z; past
      // the last block the last one is re-read.
      if (ti >= s_nrows) { ti = s_nrows - 1; u = s_nzb - 1; }
      const int r0 = ((s_tlo + ti / s_ny) * a.H + s_ylo + ti % s_ny) * a.W;
      const int z0 = s_zlo + u * KB;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        if (CHUNKS < NT && c >= CHUNKS) break;
        const int z = z0 + c / (D / 8);
        nrow[i] = r0 + (z < a.W ? z : a.W - 1);
        STA_CHECK(a.dbg, (unsigned)nrow[i] < (unsigned)a.N, 2);
      }
      return;
    }
    const int tb = kvb_l[ti < nkv ? ti : nkv - 1];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      nrow[i] = tb + off_l[u * KB + c / (D / 8)];
      if constexpr (PARTIAL) nrow[i] = nrow[i] < a.N ? nrow[i] : (int)a.N - 1;
      STA_CHECK(a.dbg, (unsigned)nrow[i] < (unsigned)a.N, 2);
      STA_CHECK(a.dbg, u * KB + c / (D / 8) < a.V, 4);
    }
  };
  // SEP: a 32-key block is read with buffer loads at a per-lane constant
  // byte offset (the chunk's position in the block) plus the block's first
  // row from the step table, looked up one fetch ahead; fetches past the
  // walk re-read its last block.
  int voff[CPT];
  const int nwalk = nkv * spt;
  if constexpr (SEP) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      voff[i] = (off_l[(c / (D / 8)) % KB] - off_l[0]) * (D * EB) + (c % (D / 8)) * 8 * EB;
    }
  }
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(kg), (short)0, SEP ? (int)(a.N * D * EB) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(vg), (short)0, SEP ? (int)(a.N * D * EB) : 0, 0x00020000);
  auto fetch = [&](Raw8<F32IN>(&dst)[CPT], const char *src, int (&nrow)[CPT], int &ti, int &u) {
    if constexpr (SEP) {
      // nrow[0] holds the byte offset of the block to fetch, ti its step
      const __amdgpu_buffer_rsrc_t rs = src == kg ? krs : vrs;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        if (CHUNKS < NT && c >= CHUNKS) break;
        // (PARTIAL: rows past the tensor are read as zeros by the buffer's
        // range check, and masked)
        STA_CHECK(a.dbg, nrow[0] >= 0 && (PARTIAL || (long long)nrow[0] + voff[i] + 8 * EB <= a.N * D * EB), 2);
        if constexpr (F32IN) {
          dst[i].x = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + nrow[0], 0, 0));
          dst[i].y = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + nrow[0] + 16, 0, 0));
        } else {
          dst[i].x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + nrow[0], 0, 0));
        }
      }
      ++ti;
      nrow[0] = stp_l[ti < nwalk ? ti : nwalk - 1];
      return;
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      dst[i] = load_raw<F32IN>(src + ((size_t)nrow[i] * D + (c % (D / 8)) * 8) * EB);
    }
    if (++u == spt) { u = 0; ++ti; }
    rows_at(nrow, ti, u);
  };
  auto stash_k = [&](const Raw8<F32IN>(&src)[CPT], int stage) {
    char *ks = smem + stage * KST_BYTES;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      *reinterpret_cast<uint4 *>(ks + (c / (D / 8)) * KSTR + (c % (D / 8)) * 16) = as_bf16<F32IN>(src[i]);
    }
  };
  // V is stored as fp16 for the P.V product.  vscale == 1: plain
  // conversion; otherwise (SCALED) V is multiplied by vscale (a power of
  // two) first.
  float vscale = 1.f;
  auto stash_v = [&](const Raw8<F32IN>(&src)[CPT], int stage) {
    char *vs = smem + 2 * KST_BYTES + stage * VST_BYTES;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      *reinterpret_cast<uint4 *>(vs + (c / (D / 8)) * VSTR + (c % (D / 8)) * 16) =
          FIXUP ? as_f16_scaled<F32IN>(src[i], vscale) : as_f16<F32IN>(src[i]);
    }
  };

  f32x4 o[DB][QB];
  float m[QB], l[QB];
  const float sl2e = a.sl2e;
  f32x4 st[2][QB];   // S^T of the current block
  f16x8 pb[QB];      // its probabilities, fp16

  // S^T[key][query] = K Q^T for 32 keys (two 16-key blocks) x 16*QB queries.
  auto qk = [&](int stage) {
    const char *ks = smem + stage * KST_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < QB; ++j) st[kb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(ks + (kb * 16 + l16) * KSTR + (32 * c + 8 * g) * 2);
#pragma unroll
        for (int j = 0; j < QB; ++j)
          st[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[j][c], st[kb][j], 0, 0, 0);
      }
    }
  };

  // PARTIAL: scores of keys that do not exist (block s of the walk) -> -inf;
  // a block whose keys all exist (every block of an interior tile) skips it.
  auto mask_block = [&](int s) {
    if constexpr (PARTIAL) {
      const uint32_t w = __builtin_amdgcn_readfirstlane(mw_l[s]);
      if (w != 0xffffffffu) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = (w >> (kb * 16 + 4 * g + r)) & 1u;
#pragma unroll
            for (int j = 0; j < QB; ++j)
              if (!ok) st[kb][j][r] = -INFINITY;
          }
      }
    }
  };

  // SWA: per lane and query block, the query's window starts; the current
  // block's key row (t, y) and z of its first key.
  int swq[QB][3];
  int cur_row = 0, cur_u = 0;
  if constexpr (SWA) {
    const int ct = qt / (a.gH * a.gW), cy = (qt / a.gW) % a.gH, cz = qt % a.gW;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int loc = qloc0 + 16 * j + l16;
      const int lt = loc / (a.tH * a.tW), ly = (loc / a.tW) % a.tH, lz = loc % a.tW;
      swq[j][0] = tok_start(ct * a.tT + lt, s_wt, a.T);
      swq[j][1] = tok_start(cy * a.tH + ly, s_wy, a.H);
      swq[j][2] = tok_start(cz * a.tW + lz, s_wz, a.W);
    }
  }
  // SWA: scores outside each query's own window -> -inf (block s, whose
  // position the step keeps in cur_row / cur_u).
  auto mask_swa = [&]() {
    if constexpr (SWA) {
      const int t = s_tlo + cur_row / s_ny, y = s_ylo + cur_row % s_ny, z0 = s_zlo + cur_u * KB;
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const bool ty = (unsigned)(t - swq[j][0]) < (unsigned)s_wt && (unsigned)(y - swq[j][1]) < (unsigned)s_wy;
        const int zr = z0 + 4 * g - swq[j][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!(ty && (unsigned)(zr + kb * 16 + r) < (unsigned)s_wz)) st[kb][j][r] = -INFINITY;
      }
    }
  };

  // In-lane max of the block in st (8 scores per query and lane).
  auto lane_max = [&](int j) {
    return fmaxf(fmaxf(fmaxf(st[0][j][0], st[0][j][1]), fmaxf(st[0][j][2], st[0][j][3])),
                 fmaxf(fmaxf(st[1][j][0], st[1][j][1]), fmaxf(st[1][j][2], st[1][j][3])));
  };
  // Probabilities of the block in st against each row's reference max m:
  // lane holds query 16j + l16, keys 4g + r and 16 + 4g + r.  They go to pb
  // in fp16; their sum over the lane's keys is added to acc.
  float mb[QB];      // m * scale * log2(e)
  auto probs = [&](int j, float &acc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][j][r], sl2e, -mb[j]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][j][r + 1], sl2e, -mb[j]));
        const f16x2 pp = f16x2{(_Float16)p0, (_Float16)p1};
        pb[j][kb * 4 + r] = pp[0];
        pb[j][kb * 4 + r + 1] = pp[1];
        acc = __builtin_amdgcn_fdot2(pp, f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
      }
  };
  // Softmax of one block.  The new row sums are checked before they replace
  // l: an overflowed probability makes its row sum +inf, and then the wave
  // repairs the block: every row's reference rises to 2^4 (exp2 units)
  // above the row's max so far unless it is higher already, O and l are
  // rescaled and the block's probabilities recomputed (a row whose reference
  // moved now has them all <= 2^-4).  The headroom lets a row's max grow by
  // 2^20 instead of 2^16 before the next repair: on inputs whose
  // rows' maxima keep growing along the walk (per-token magnitudes up to 4)
  // it removes a fifth of the repairs, each of which holds the work group
  // at the step's barrier, and keeps the probabilities within fp16's normal
  // range relative to the row's largest.  O is in VGPRs, so the rescale
  // needs no register copies.
  auto softmax = [&]() {
    float ln[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      ln[j] = l[j];
      probs(j, ln[j]);
    }
    float lmax = ln[0];
#pragma unroll
    for (int j = 1; j < QB; ++j) lmax = fmaxf(lmax, ln[j]);
    if (__builtin_amdgcn_ballot_w64(!(lmax <= 3.0e38f))) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const float mnew = fmaxf(m[j], swap_max(lane_max(j)) + 4.f / sl2e);
        const float alpha = __builtin_amdgcn_exp2f((m[j] - mnew) * sl2e);
        m[j] = mnew;
        mb[j] = mnew * sl2e;
        ln[j] = l[j] * alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b) o[b][j] *= alpha;
        probs(j, ln[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) l[j] = ln[j];
  };

  // O^T[d][query] += V^T P^T.
  const int trow = 4 * g + (l16 >> 2);
  const int tcol = 4 * (l16 & 3);
  auto pvmm = [&](int stage) {
    const char *vs = smem + 2 * KST_BYTES + stage * VST_BYTES;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const lds_char *vb = (const lds_char *)(vs) + b * 32 + tcol * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vb + trow * VSTR));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vb + (trow + 16) * VSTR));
      f16x8 va;
      const f16x4 lob = __builtin_bit_cast(f16x4, lo), hib = __builtin_bit_cast(f16x4, hi);
      va[0] = lob[0]; va[1] = lob[1]; va[2] = lob[2]; va[3] = lob[3];
      va[4] = hib[0]; va[5] = hib[1]; va[6] = hib[2]; va[7] = hib[3];
#pragma unroll
      for (int j = 0; j < QB; ++j) o[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[j], o[b][j], 0, 0, 0);
    }
  };

  // Ping-pong: the two waves sharing a SIMD (w and w + NW/2) run the step in
  // opposite orders, so one wave's softmax VALU work overlaps the other's
  // MFMAs:
  //   group A  PV(s-1), QK(s), softmax(s)
  //   group B  softmax(s-1), PV(s-1), QK(s)
  // LDS holds K(s) and V(s-1) during step s; K(s+1) and V(s) are written
  // into the other LDS stages at its end, followed by the step's only
  // barrier.  They come from registers loaded one step earlier: two register
  // buffers alternate, so a block's global loads have a whole step to
  // arrive (with loads issued in the step that writes them, the waits for
  // them at the step's end cost about a tenth of the kernel's time on
  // MI355X).  Measured on MI355X as well: this beat a barrier between the
  // halves, per-group LDS writes inside the softmax half, and loads by one
  // group only.
  // (grp_a is uniform across a wave.  Telling the compiler so with
  // readfirstlane turns the two orders into scalar branches but makes the
  // register allocation spill.)
  const bool grp_a = wave < NW / 2;
  // Start of the walk over the key blocks: K(0) in LDS stage 0, V stage 1
  // zeroed (step 0's P.V of the nonexistent block -1 reads it, with zero
  // probabilities).
  auto begin_walk = [&]() {
    fk_ti = fv_ti = s_first / spt;
    fk_u = fv_u = s_first % spt;
    if constexpr (SWA) { cur_row = 0; cur_u = 0; }
    if constexpr (SEP) {
      // the step counters live in fk_ti / fv_ti, the table offsets in krow[0] / vrow[0]
      fk_ti = fv_ti = s_first;
      krow[0] = vrow[0] = stp_l[s_first];
    } else {
      rows_at(krow, fk_ti, fk_u);
      rows_at(vrow, fv_ti, fv_u);
    }
    fetch(rk, kg, krow, fk_ti, fk_u);
    stash_k(rk, 0);
    uint4 *v1 = reinterpret_cast<uint4 *>(smem + 2 * KST_BYTES + VST_BYTES);
    for (int i = tid; i < VST_BYTES / 16; i += NT) v1[i] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    // Retire every outstanding load (the Q fragments included) before the
    // loop, so that inside it the only vector-memory waits are the ones for
    // the prefetched K/V blocks at their LDS writes.
    __builtin_amdgcn_s_waitcnt(0);
  };

  // fp16 holds |v| <= 65504.  A V entry beyond it becomes an infinity in
  // the P.V operand, which makes the work group's O non-finite; with finite
  // inputs nothing else can (the probabilities are fp16 too, and a row sum
  // that overflows is repaired before it is used, so |O| <= 65504^2 times
  // the keys' count).  The check runs on the accumulators' bits as
  // integers: their exponent field is all ones only for an infinity or a
  // NaN (a floating-point test would be folded away, since this file is
  // built without NaN semantics).  A wave that finds one marks its item
  // (once per item, through a bit set), and the launch's second kernel
  // (FIXUP) redoes every marked item with V multiplied by 2^-e, e chosen
  // from the largest |v| of the item's keys, and O by 2^e: exact scalings,
  // so only fp16's range moves (entries below 2^(e-25) of the largest round
  // to zero, far below the output's precision).  No barrier is added to the
  // common path.
  float oscale = 1.f;
  if constexpr (FIXUP) {
    if (tid == 0) vmax_bits = 0u;
    fv_ti = s_first / spt;
    fv_u = s_first % spt;
    if constexpr (SEP) {
      fv_ti = s_first;
      vrow[0] = stp_l[s_first];
    } else {
      rows_at(vrow, fv_ti, fv_u);
    }
    float vm = 0.f;
    for (int s = 0; s < nsteps; ++s) {
      fetch(rv, vg, vrow, fv_ti, fv_u);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        if (CHUNKS < NT && c >= CHUNKS) break;
        vm = fmaxf(vm, max_abs8<F32IN>(rv[i]));
      }
    }
    __syncthreads();
    atomicMax(&vmax_bits, __float_as_uint(vm));
    __syncthreads();
    int ex = 0;
    (void)frexpf(__uint_as_float(vmax_bits), &ex);   // largest |v| < 2^ex
    const int e = ex > 15 ? ex - 15 : 0;              // largest |v| * 2^-e < 2^15
    vscale = ldexpf(1.f, -e);
    oscale = ldexpf(1.f, e);
  }

  // The walk: the initial reference max, then every key block of this
  // work group's steps.
  begin_walk();
  // Initial reference max: each row's max over the first key block (which
  // always holds an existing key: a tile's first token is inside the video).
  // SWA: the query's score against its own key.
  if constexpr (SWA) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int row = qbase + off_l[qloc0 + 16 * j + l16];
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 kx = __builtin_bit_cast(bf16x8, as_bf16<F32IN>(load_raw<F32IN>(
                                                 kg + ((size_t)row * D + 32 * c + 8 * g) * EB)));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)qf[j][c][e], (float)kx[e], acc);
      }
      m[j] = swap_sum(acc);
    }
  } else {
    qk(0);
    mask_block(s_first);
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if constexpr (!SWA) m[j] = swap_max(lane_max(j));
    mb[j] = m[j] * sl2e;
    l[j] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Group B's softmax of block -1 at step 0 must give zero probabilities,
    // and group A's P.V of block -1 must add nothing.
    pb[j] = f16x8{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) st[kb][j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }

  // The loop has no other branches than the group's order (and the odd
  // step count's end): fetches past the last block re-read the last key
  // tile and are written to a stage nobody reads again.
  Raw8<F32IN> rk2[CPT], rv2[CPT];
  fetch(rk, kg, krow, fk_ti, fk_u);   // K(1)
  fetch(rv, vg, vrow, fv_ti, fv_u);   // V(0)
  auto step = [&](int s, Raw8<F32IN>(&ck)[CPT], Raw8<F32IN>(&cv)[CPT], Raw8<F32IN>(&nk)[CPT],
                  Raw8<F32IN>(&nv)[CPT]) {
    fetch(nk, kg, krow, fk_ti, fk_u);   // K(s+2)
    fetch(nv, vg, vrow, fv_ti, fv_u);   // V(s+1)
    if (grp_a) {
      pvmm((s - 1) & 1);
      qk(s & 1);
      mask_block(s_first + s);
      mask_swa();
    } else {
      softmax();
    }
    if (grp_a) {
      softmax();
    } else {
      pvmm((s - 1) & 1);
      qk(s & 1);
      mask_block(s_first + s);
      mask_swa();
    }
    if constexpr (SWA) {
      if (++cur_u == s_nzb) { cur_u = 0; ++cur_row; }
    }
    stash_k(ck, (s + 1) & 1);
    stash_v(cv, s & 1);
    __syncthreads();
  };
  // An odd last step runs after the loop: with it inside (a conditional
  // second step), the path that skips it returns to the loop head with the
  // first step's loads still outstanding, and the compiler's wait for them
  // at the head then also retired every iteration's newest loads.
  for (int s = 0; s + 1 < nsteps; s += 2) {
    step(s, rk, rv, rk2, rv2);
    step(s + 1, rk2, rv2, rk, rv);
  }
  if (nsteps & 1) step(nsteps - 1, rk, rv, rk2, rv2);
  if (!grp_a) softmax();
  pvmm((nsteps - 1) & 1);
  if constexpr (!FIXUP) {
    unsigned top = 0u;   // largest (bits << 1): exponent field all ones iff >= 0xff000000
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) top = max(top, __float_as_uint(o[b][j][r]) << 1);
    if (__builtin_amdgcn_ballot_w64(top >= 0xff000000u) != 0 && lane == 0) {
      const unsigned bit = 1u << (item & 31);
      if (!(atomicOr(a.fbits + (item >> 5), bit) & bit)) a.flist[atomicAdd(a.qcount + 11, 1)] = item;
    }
  }

  // ---- a piece of a split item: publish the partial result (unnormalised
  // O, reference maxima and row-sum partials); the group's last piece to
  // arrive combines all of them and finalizes (with per-work-group lists, a
  // piece that starts its publication after every other one has arrived
  // skips it).  Softmax pieces combine
  // exactly: with M = max of the pieces' reference maxima (exp2 units),
  // O = sum_p 2^(mb_p - M) O_p and l = sum_p 2^(mb_p - M) l_p.  Pieces may
  // run on different XCDs, whose L2 caches are not coherent with each
  // other: the partial result is released with one agent-scope fence (L2
  // write-back) per work group after every wave's stores have completed,
  // and the last piece acquires with one agent-scope fence (L2
  // invalidation) before reading.  One fence per work group rather than one
  // per wave: each writes back or invalidates the whole L2 of the XCD, which
  // slows every work group on it.
  if (piece >= 0) {
    if constexpr (!SWA && QB == 3 && NW == 8) {
      if (oscale != 1.f) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int j = 0; j < QB; ++j) o[b][j] *= oscale;
        oscale = 1.f;
      }
      if constexpr (MULTI) {
        // Per-work-group lists: a piece that finds every other one of its
        // group arrived skips its publication.  Kept apart from the section
        // below, which the large launches run: there the same source with a
        // run-time branch cost 1 % through code layout.
        constexpr int SLOT = 384 * D + 2 * QB * NT;   // floats per slot (fwd_slot_floats)
        constexpr int ML = DB * QB * NT * 4;           // float offset of the maxima and row sums
        const int group = __builtin_amdgcn_readfirstlane(a.ptab[4 * piece + 3]);
        const int first = __builtin_amdgcn_readfirstlane(a.gtab[2 * group]);
        const int np = __builtin_amdgcn_readfirstlane(a.gtab[2 * group + 1]);
        // A piece that finds every other piece of its group arrived is the
        // last: it publishes nothing and keeps its own partial in registers
        // (acquire: the relaxed load that saw the count, then a fence).
        if (tid == 0) {
          const bool all =
              __hip_atomic_load(a.pcount + group, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
          if (all) {
            __threadfence();                                 // acquire
            atomicExch(a.pcount + group, 0);                 // ready for the next launch
          }
          last_piece = all ? 2 : 0;
        }
        __syncthreads();
        if (last_piece == 0) {
          float *slot = a.pslot + (size_t)piece * SLOT;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int j = 0; j < QB; ++j) reinterpret_cast<f32x4 *>(slot)[(b * QB + j) * NT + tid] = o[b][j];
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            slot[ML + j * NT + tid] = mb[j];
            slot[ML + (QB + j) * NT + tid] = l[j];
          }
          // Every wave's stores have reached its XCD's L2 before the release.
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (tid == 0) {
            __threadfence();                                 // release
            const bool last = atomicAdd(a.pcount + group, 1) == np - 1;
            if (last) {
              __threadfence();                               // acquire
              atomicExch(a.pcount + group, 0);               // ready for the next launch
            }
            last_piece = last;
          }
          __syncthreads();
          if (!last_piece) {
            __syncthreads();
            goto next_item;
          }
        }
        // Combined in piece order as below, the own partial taken from
        // registers (the same values as its published copy).
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          float mx = -INFINITY;
          for (int p = first; p < first + np; ++p)
            mx = fmaxf(mx, p == piece ? mb[j] : a.pslot[(size_t)p * SLOT + ML + j * NT + tid]);
          float lj = 0.f;
          f32x4 oj[DB];
#pragma unroll
          for (int b = 0; b < DB; ++b) oj[b] = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int p = first; p < first + np; ++p) {
            if (p == piece) {
              const float f = __builtin_amdgcn_exp2f(mb[j] - mx);
              lj += f * l[j];
#pragma unroll
              for (int b = 0; b < DB; ++b) oj[b] += f * o[b][j];
            } else {
              const float *slot = a.pslot + (size_t)p * SLOT;
              const float f = __builtin_amdgcn_exp2f(slot[ML + j * NT + tid] - mx);
              lj += f * slot[ML + (QB + j) * NT + tid];
#pragma unroll
              for (int b = 0; b < DB; ++b) oj[b] += f * reinterpret_cast<const f32x4 *>(slot)[(b * QB + j) * NT + tid];
            }
          }
          mb[j] = mx;
          l[j] = lj;
#pragma unroll
          for (int b = 0; b < DB; ++b) o[b][j] = oj[b];
        }
      } else {
        constexpr int SLOT = 384 * D + 2 * QB * NT;   // floats per slot (fwd_slot_floats)
        constexpr int ML = DB * QB * NT * 4;           // float offset of the maxima and row sums
        {
          float *slot = a.pslot + (size_t)piece * SLOT;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int j = 0; j < QB; ++j) reinterpret_cast<f32x4 *>(slot)[(b * QB + j) * NT + tid] = o[b][j];
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            slot[ML + j * NT + tid] = mb[j];
            slot[ML + (QB + j) * NT + tid] = l[j];
          }
        }
        // Every wave's stores have reached its XCD's L2 before the release.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int group = __builtin_amdgcn_readfirstlane(a.ptab[4 * piece + 3]);
        const int first = __builtin_amdgcn_readfirstlane(a.gtab[2 * group]);
        const int np = __builtin_amdgcn_readfirstlane(a.gtab[2 * group + 1]);
        if (tid == 0) {
          __threadfence();                                   // release
          const bool last = atomicAdd(a.pcount + group, 1) == np - 1;
          if (last) {
            __threadfence();                                 // acquire
            atomicExch(a.pcount + group, 0);                 // ready for the next launch
          }
          last_piece = last;
        }
        __syncthreads();
        if (!last_piece) {
          finish();
          return;
        }
        // Combined in piece order, every partial read back (the last piece's
        // own included), so that the result does not depend on which piece
        // arrived last; one query block at a time, which keeps the loads of
        // one partial block beside the accumulators in registers.
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          float mx = -INFINITY;
          for (int p = first; p < first + np; ++p) mx = fmaxf(mx, a.pslot[(size_t)p * SLOT + ML + j * NT + tid]);
          float lj = 0.f;
          f32x4 oj[DB];
#pragma unroll
          for (int b = 0; b < DB; ++b) oj[b] = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int p = first; p < first + np; ++p) {
            const float *slot = a.pslot + (size_t)p * SLOT;
            const float f = __builtin_amdgcn_exp2f(slot[ML + j * NT + tid] - mx);
            lj += f * slot[ML + (QB + j) * NT + tid];
#pragma unroll
            for (int b = 0; b < DB; ++b) oj[b] += f * reinterpret_cast<const f32x4 *>(slot)[(b * QB + j) * NT + tid];
          }
          mb[j] = mx;
          l[j] = lj;
#pragma unroll
          for (int b = 0; b < DB; ++b) o[b][j] = oj[b];
        }
      }
    }
  }

  // ---- finalize: O = O^T / l, stored row-major; optionally the row
  // log-sum-exp, ln(sum_j exp(scale s_j)) = (m * scale * log2(e) + log2(l)) * ln(2).
  char *og = reinterpret_cast<char *>(a.o) + (size_t)bh * a.N * D * (F32OUT ? 4 : 2);
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float lsum = swap_sum(l[j]);
    const float inv = oscale / lsum;
    const int row = qbase + off_l[qloc0 + 16 * j + l16];
    if constexpr (PARTIAL) {
      const int ql = qloc0 + 16 * j + l16;
      if (!((a.kmask[(size_t)qt * spt + ql / 32] >> (ql % 32)) & 1u)) continue;
    }
    STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 3);
    if (a.lse != nullptr && g == 0)
      a.lse[(size_t)bh * a.N + row] = (mb[j] + log2f(lsum)) * 0.69314718055994530942f;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const f32x4 r = o[b][j] * inv;
      const size_t e = (size_t)row * D + b * 16 + 4 * g;
      if constexpr (F32OUT) {
        *reinterpret_cast<f32x4 *>(og + e * 4) = r;
      } else {
        bf16x4 rb;
        rb[0] = (__bf16)r[0]; rb[1] = (__bf16)r[1]; rb[2] = (__bf16)r[2]; rb[3] = (__bf16)r[3];
        *reinterpret_cast<bf16x4 *>(og + e * 2) = rb;
      }
    }
  }
  if constexpr (FIXUP || MULTI) {
    __syncthreads();
    goto next_item;
  } else {
    finish();
  }
}


__global__ void zero_kernel(int32_t *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

template <int D, int QB, int NW, bool FI, bool FO, bool PARTIAL, bool SWA, bool SEP, bool FIXUP,
          bool MULTI = false>
hipError_t launch_kernel(const FwdArgs &a, int blocks, hipStream_t s) {
  auto kern = sta_fwd_kernel<D, QB, NW, FI, FO, PARTIAL, SWA, SEP, FIXUP, MULTI>;
  const size_t lds = (size_t)fwd_lds_bytes(D, a.V, a.max_nkv) +
                     ((PARTIAL ? 1 : 0) + (SEP ? 1 : 0)) * (size_t)fwd_lds_step_bytes(a.V, a.max_nkv);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

// The forward launch, then the fix-up launch (256 work groups, which exit
// at once unless the forward marked work items whose V exceeds fp16's
// range; those are redone with V scaled).  The fix-up kernel addresses K
// and V through the tile tables (SEP off): it is the rare path.
template <int D, int QB, int NW, bool FI, bool FO, bool PARTIAL, bool SWA = false, bool SEP = false>
hipError_t launch_one(const FwdArgs &a, hipStream_t s) {
  hipError_t e;
  if constexpr (!SWA && QB == 3 && NW == 8) {
    e = a.wlist != nullptr ? launch_kernel<D, QB, NW, FI, FO, PARTIAL, SWA, SEP, false, true>(a, a.n_blocks, s)
                           : launch_kernel<D, QB, NW, FI, FO, PARTIAL, SWA, SEP, false>(a, a.n_blocks, s);
  } else {
    e = launch_kernel<D, QB, NW, FI, FO, PARTIAL, SWA, SEP, false>(a, a.n_blocks, s);
  }
  if (e != hipSuccess) return e;
  return launch_kernel<D, QB, NW, FI, FO, PARTIAL, SWA, false, true>(a, 256, s);
}

template <int D, int QB, int NW, bool P, bool SEP = false>
hipError_t launch_io(const FwdArgs &a, bool f32_in, bool f32_out, hipStream_t s) {
  if (f32_in)
    return f32_out ? launch_one<D, QB, NW, true, true, P, false, SEP>(a, s)
                   : launch_one<D, QB, NW, true, false, P, false, SEP>(a, s);
  return f32_out ? launch_one<D, QB, NW, false, true, P, false, SEP>(a, s)
                 : launch_one<D, QB, NW, false, false, P, false, SEP>(a, s);
}

template <int D, int QB, int NW>
hipError_t launch_p(const FwdArgs &a, bool f32_in, bool f32_out, hipStream_t s) {
  if (a.swin != nullptr) {
    if (f32_in) return f32_out ? launch_one<D, QB, NW, true, true, false, true>(a, s)
                               : launch_one<D, QB, NW, true, false, false, true>(a, s);
    return f32_out ? launch_one<D, QB, NW, false, true, false, true>(a, s)
                   : launch_one<D, QB, NW, false, false, false, true>(a, s);
  }
  if (a.kmask != nullptr) {
    if (a.sep) return launch_io<D, QB, NW, true, true>(a, f32_in, f32_out, s);
    return launch_io<D, QB, NW, true>(a, f32_in, f32_out, s);
  }
  if (a.sep) return launch_io<D, QB, NW, false, true>(a, f32_in, f32_out, s);
  return launch_io<D, QB, NW, false>(a, f32_in, f32_out, s);
}

}  // namespace

hipError_t launch_zero(int32_t *p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs &a, int variant, int head_dim, bool f32_in, bool f32_out,
                          hipStream_t stream) {
  if (a.n_blocks <= 0) return hipSuccess;
  // Split items and per-group lists exist only for the 384-query kernel
  // (not token-wise SWA).
  if ((a.ptab != nullptr || a.wlist != nullptr) && (variant != kTile384 || a.swin != nullptr))
    return hipErrorInvalidValue;
  if (variant == kTile384) {
    if (head_dim == 128) return launch_p<128, 3, 8>(a, f32_in, f32_out, stream);
    return launch_p<64, 3, 8>(a, f32_in, f32_out, stream);
  }
  if (head_dim == 128) return launch_p<128, 1, 2>(a, f32_in, f32_out, stream);
  return launch_p<64, 1, 2>(a, f32_in, f32_out, stream);
}

}  // namespace sta
