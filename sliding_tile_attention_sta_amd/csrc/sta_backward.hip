// Sliding Tile Attention backward for gfx950 (MI355X).
//
// The pages fine-tune the video model with STA in place ("Fast Video
// Generation with Sliding Tile Attention", arXiv 2502.04507, index page,
// Abstract; gptget summary page, Summary and Experiments), so the operator is
// trained through.  Its gradients are those of softmax attention restricted
// to each query tile's window (chain rule of the forward definition):
//
//   P_ij  = exp(scale q_i.k_j - lse_i)        (lse from the forward)
//   dv_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i.v_j - delta_i),        delta_i = dO_i . O_i
//   dq_i  = scale sum_j dS_ij k_j,            dk_j = scale sum_i dS_ij q_i
//
// As in the forward, whole (query tile, key tile) pairs are attended or
// skipped, so no kernel evaluates a mask.  Three kernels, no atomics (the
// result does not depend on scheduling):
//
//   * delta: one fused multiply-add pass over dO and O (HBM bound).
//   * dQ: a work group owns 32*NW queries of one (batch, head, query tile)
//     and walks the key tiles of its window, 32 keys per step, like the
//     forward: S^T = K Q^T and dP^T = V dO^T with the queries' Q and dO in
//     VGPRs, then dQ^T += K^T dS^T with K^T read from LDS by the transposing
//     ds_read_b64_tr_b16.
//   * dK/dV: a work group owns 32*NW keys of one (batch, head, key tile) and
//     walks the query tiles whose window holds that key tile (the inverse
//     lists of the plan), 32 queries per step: S = Q K^T and dP = dO V^T with
//     the keys' K and V in VGPRs, then dV^T += dO^T P and dK^T += Q^T dS with
//     dO^T and Q^T read transposed from LDS.
//
// Extents that are not multiples of the tile (partial tiles at the far
// edges; a separate instantiation of each kernel, PARTIAL): as in the
// forward, only tokens that exist take part.  Rows of tile positions that
// do not exist are clamped to the tensor for loading, the walk's validity
// words (one per 32-token block, staged in LDS) zero dS of keys that do
// not exist (dQ) and give queries that do not exist an infinite log-sum-
// exp, so their P and dS are 0 (dK/dV), and nothing is stored for them;
// such a row's own gradient is computed from clamped values and dropped.
//
// The products run on v_mfma_f32_16x16x32_f16 with fp32 accumulation.
// P and dS are rounded to fp16 (11 significant bits against bf16's 8); Q and
// K are the forward's bf16 values (fp32 inputs rounded to bf16 first, so
// that the scores match the ones the forward's lse was taken over), widened
// to fp16, which is exact inside the fp16 range; V and dO are converted to
// fp16 (exact for bf16 values inside the range, nearest-even for fp32).  One
// exception: with bf16 inputs the dQ kernel's dP^T = V dO^T takes V and dO
// as they are on v_mfma_f32_16x16x32_bf16 (the same exact products, without
// the per-step conversion of V).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"
#include "sta_launch.h"

namespace sta {
namespace {

constexpr int TB = kKeyBlock;  // tokens per pipeline step (keys for dQ, queries for dK/dV)
constexpr float kLog2e = 1.44269504088896340736f;

// Q and K chunks as fp16 holding the forward's bf16 values.
template <bool F32>
__device__ __forceinline__ uint4 score_f16(const Raw8<F32> &r) {
  if constexpr (F32) {
    Raw8<false> b;
    b.x = as_bf16<true>(r);
    return as_f16<false>(b);
  } else {
    return as_f16<false>(r);
  }
}

__device__ __forceinline__ f16x8 lds_f16x8(const char *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ bf16x8 lds_bf16x8(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// V and dO for the dQ kernel's dP^T: bf16 chunks as they are, fp32 chunks
// converted to fp16.
template <bool F32>
__device__ __forceinline__ uint4 dp_operand(const Raw8<F32> &r) {
  if constexpr (F32) return as_f16<true>(r);
  else return r.x;
}

// Transposed 16x16x32 operand from a row-major fp16 [32][*] LDS block: lane
// (g, l16) receives column col0 + l16 of rows 4g..4g+3 (slots 0..3) and
// 16+4g..16+4g+3 (slots 4..7).  The same slot order is used for the
// register operand it is multiplied with.
__device__ __forceinline__ f16x8 lds_tr(const char *blk, int stride, int col0, int trow, int tcol) {
  const lds_char *b = (const lds_char *)(blk) + (col0 + tcol) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(b + trow * stride));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(b + (trow + 16) * stride));
  const f16x4 l = __builtin_bit_cast(f16x4, lo), h = __builtin_bit_cast(f16x4, hi);
  return f16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

__device__ __forceinline__ void store4(void *base, size_t e, const f32x4 &r, bool f32) {
  if (f32) {
    *reinterpret_cast<f32x4 *>(static_cast<char *>(base) + e * 4) = r;
  } else {
    bf16x4 b;
    b[0] = (__bf16)r[0]; b[1] = (__bf16)r[1]; b[2] = (__bf16)r[2]; b[3] = (__bf16)r[3];
    *reinterpret_cast<bf16x4 *>(static_cast<char *>(base) + e * 2) = b;
  }
}

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O): D/8 lanes per row, 8 elements per lane; a
// block-uniform grid-stride loop, so the shuffles always see whole rows.
// ---------------------------------------------------------------------------
template <int D, bool F32O, bool F32G>
__global__ __launch_bounds__(256) void sta_bwd_delta_kernel(const void *o, const void *g, float *delta,
                                                            int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t total = rows * LPR;
  for (int64_t t0 = (int64_t)blockIdx.x * 256; t0 < total; t0 += (int64_t)gridDim.x * 256) {
    const int64_t t = t0 + threadIdx.x;
    const int64_t row = t / LPR;
    const int c = (int)(t % LPR);
    float acc = 0.f;
    if (row < rows) {
      const size_t e = (size_t)row * D + c * 8;
      float ov[8], gv[8];
      if constexpr (F32O) {
        const float4 a = reinterpret_cast<const float4 *>(static_cast<const float *>(o) + e)[0];
        const float4 b = reinterpret_cast<const float4 *>(static_cast<const float *>(o) + e)[1];
        ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w; ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
      } else {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(o) + e);
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] = (float)a[i];
      }
      if constexpr (F32G) {
        const float4 a = reinterpret_cast<const float4 *>(static_cast<const float *>(g) + e)[0];
        const float4 b = reinterpret_cast<const float4 *>(static_cast<const float *>(g) + e)[1];
        gv[0] = a.x; gv[1] = a.y; gv[2] = a.z; gv[3] = a.w; gv[4] = b.x; gv[5] = b.y; gv[6] = b.z; gv[7] = b.w;
      } else {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(g) + e);
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = (float)a[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(ov[i], gv[i], acc);
    }
#pragma unroll
    for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
    if (row < rows && c == 0) delta[row] = acc;
  }
}

// Work item decode shared by both kernels: (batch*heads + h, tile, sub).
struct Item {
  int sub, tile, bh, h;
};
__device__ __forceinline__ Item decode(int item, const BwdArgs &a) {
  Item it;
  it.sub = item % a.subs;
  const int rest = item / a.subs;
  it.tile = rest % a.n_tiles;
  it.bh = rest / a.n_tiles;
  it.h = it.bh % a.heads;
  return it;
}

// PARTIAL (extents that are not multiples of the tile): a tile-local token
// that does not exist has a row past the tile's edge, possibly past the
// tensor; loads take the last row instead (their values are masked), and
// nothing is stored for it.  exists(): bit (local mod 32) of the tile's
// validity word (local / 32).
template <bool PARTIAL>
__device__ __forceinline__ int clamp_row(int row, int64_t n) {
  if constexpr (PARTIAL) return row < n ? row : (int)n - 1;
  return row;
}
__device__ __forceinline__ bool exists(const uint32_t *kmask, int tile, int local, int V) {
  return (kmask[(size_t)tile * (V / TB) + local / TB] >> (local % TB)) & 1u;
}

// ---------------------------------------------------------------------------
// dQ: queries resident, key blocks streamed.
// ---------------------------------------------------------------------------
template <int D, int NW, bool F32IN, bool PARTIAL>
// Two waves per SIMD: without the hint the allocator parks the Q and dO
// fragments in AGPRs and copies them back every step (about 100 extra VALU
// instructions per step).  Except for one wave with D = 128 (tile volumes
// that are not a multiple of 128): it stages 8 chunks of K and of V per
// step, which does not fit in 256 VGPRs, and the AGPRs are the place to
// spill to (with the hint it spilled to scratch).
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(NW == 1 && D == 128 ? 1 : 2, 2))) void sta_bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int QPI = 32 * NW;
  constexpr int STR = bwd_stride(D);
  constexpr int ST = TB * STR;                   // bytes of one stage of one tensor
  constexpr int CHUNKS = TB * D / 8;
  constexpr int CPT = (CHUNKS + NT - 1) / NT;
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "chunk split");
  constexpr int EB = F32IN ? 4 : 2;
  constexpr int DC = D / 32;
  constexpr int DB = D / 16;

  // LDS: K stages 0/1, V stages 0/1, tile-local offsets, key-tile base rows
  // (PARTIAL: then the validity word of every 32-key block of the walk).
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int *off_l = reinterpret_cast<int *>(smem + 4 * ST);
  int *lb_l = off_l + a.V;
  uint32_t *mw_l = reinterpret_cast<uint32_t *>(lb_l + a.max_list);

  const int item = __builtin_amdgcn_readfirstlane(a.sched[blockIdx.x]);
  if (item < 0) return;
  STA_CHECK(a.dbg, item < a.n_items, 0);
  const Item it = decode(item, a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  const int l0 = __builtin_amdgcn_readfirstlane(a.list_off[it.h * a.n_tiles + it.tile]);
  const int nl = __builtin_amdgcn_readfirstlane(a.list_off[it.h * a.n_tiles + it.tile + 1]) - l0;
  for (int i = tid; i < a.V; i += NT) off_l[i] = a.off[i];
  for (int i = tid; i < nl; i += NT) {
    STA_CHECK(a.dbg, (unsigned)a.list_idx[l0 + i] < (unsigned)a.n_tiles && i < a.max_list, 1);
    lb_l[i] = a.base[a.list_idx[l0 + i]];
  }
  if constexpr (PARTIAL) {
    const int words = a.V / TB;
    for (int i = tid; i < nl * words; i += NT) mw_l[i] = a.kmask[(size_t)a.list_idx[l0 + i / words] * words + i % words];
  }

  const size_t plane = (size_t)it.bh * a.N;
  const char *qg = static_cast<const char *>(a.q) + plane * D * EB;
  const char *kg = static_cast<const char *>(a.k) + plane * D * EB;
  const char *vg = static_cast<const char *>(a.v) + plane * D * EB;
  const char *gg = static_cast<const char *>(a.dout) + plane * D * EB;
  const int qbase = a.base[it.tile];
  const int qloc0 = it.sub * QPI + wave * 32;
  __syncthreads();

  // Q and dO of the wave's 32 queries (B operands; lane: query 16j + l16).
  using DpT = typename std::conditional<F32IN, f16x8, bf16x8>::type;
  f16x8 qf[2][DC];
  DpT gf[2][DC];
  float lse2[2], dl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = clamp_row<PARTIAL>(qbase + off_l[qloc0 + 16 * j + l16], a.N);
    STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 2);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const size_t e = (size_t)row * D + 32 * c + 8 * g;
      qf[j][c] = __builtin_bit_cast(f16x8, score_f16<F32IN>(load_raw<F32IN>(qg + e * EB)));
      gf[j][c] = __builtin_bit_cast(DpT, dp_operand<F32IN>(load_raw<F32IN>(gg + e * EB)));
    }
    lse2[j] = a.lse[plane + row] * kLog2e;
    dl[j] = a.delta[plane + row];
  }

  const int spt = a.V / TB;
  const int nsteps = nl * spt;
  // K/V chunks pass through two register buffers: block s+2 is loaded at
  // the start of step s into one while the other (block s+1, loaded a step
  // earlier) is written to LDS at its end, so every block's loads have a
  // whole step to arrive.  Loads past the last block re-read it, into a
  // stage nobody reads again.
  Raw8<F32IN> rka[CPT], rva[CPT], rkb[CPT], rvb[CPT];
  auto fetch = [&](int s, Raw8<F32IN>(&dk)[CPT], Raw8<F32IN>(&dv)[CPT]) {
    if (s > nsteps - 1) s = nsteps - 1;
    const int tb = lb_l[s / spt], u = s % spt;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      const int row = clamp_row<PARTIAL>(tb + off_l[u * TB + c / (D / 8)], a.N);
      STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 2);
      const size_t e = (size_t)row * D + (c % (D / 8)) * 8;
      dk[i] = load_raw<F32IN>(kg + e * EB);
      dv[i] = load_raw<F32IN>(vg + e * EB);
    }
  };
  auto stash = [&](const Raw8<F32IN>(&sk)[CPT], const Raw8<F32IN>(&sv)[CPT], int stage) {
    char *ks = smem + stage * ST, *vs = smem + (2 + stage) * ST;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      const int o = (c / (D / 8)) * STR + (c % (D / 8)) * 16;
      *reinterpret_cast<uint4 *>(ks + o) = score_f16<F32IN>(sk[i]);
      *reinterpret_cast<uint4 *>(vs + o) = dp_operand<F32IN>(sv[i]);
    }
  };

  f32x4 acc[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2e = a.sl2e;
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);

  if (nsteps > 0) {
    fetch(0, rka, rva);
    stash(rka, rva, 0);
    fetch(1, rka, rva);
  }
  __syncthreads();
  auto step = [&](int s, const Raw8<F32IN>(&ck)[CPT], const Raw8<F32IN>(&cv)[CPT], Raw8<F32IN>(&nk)[CPT],
                  Raw8<F32IN>(&nv)[CPT]) {
    fetch(s + 2, nk, nv);
    const char *ks = smem + (s & 1) * ST, *vs = smem + (2 + (s & 1)) * ST;
    // S^T = K Q^T, dP^T = V dO^T; lane: query 16j + l16, keys 16kb + 4g + r.
    f32x4 st[2][2], dp[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        st[kb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int o = (kb * 16 + l16) * STR + (32 * c + 8 * g) * 2;
        const f16x8 ka = lds_f16x8(ks + o);
#pragma unroll
        for (int j = 0; j < 2; ++j) st[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[j][c], st[kb][j], 0, 0, 0);
        if constexpr (F32IN) {
          const f16x8 va = lds_f16x8(vs + o);
#pragma unroll
          for (int j = 0; j < 2; ++j) dp[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, gf[j][c], dp[kb][j], 0, 0, 0);
        } else {
          const bf16x8 va = lds_bf16x8(vs + o);
#pragma unroll
          for (int j = 0; j < 2; ++j) dp[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, gf[j][c], dp[kb][j], 0, 0, 0);
        }
      }
    // dS^T in fp16, slots: keys 4g + r (kb 0) and 16 + 4g + r (kb 1).
    // PARTIAL: keys that do not exist get dS = 0 (a block whose keys all
    // exist, every block of an interior tile, skips it on a scalar branch).
    f16x8 dsf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][j][r], sl2e, -lse2[j]));
          dsf[j][kb * 4 + r] = (_Float16)(p * (dp[kb][j][r] - dl[j]));
        }
    if constexpr (PARTIAL) {
      const uint32_t kw = __builtin_amdgcn_readfirstlane(mw_l[s]);
      if (kw != 0xffffffffu) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (!((kw >> (kb * 16 + 4 * g + r)) & 1u)) dsf[j][kb * 4 + r] = (_Float16)0.f;
      }
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const f16x8 kt = lds_tr(ks, STR, 16 * b, trow, tcol);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt, dsf[j], acc[b][j], 0, 0, 0);
    }
    stash(ck, cv, (s + 1) & 1);
    __syncthreads();
  };
  // Two steps per iteration (the buffers alternate); an odd last step runs
  // after the loop, so that no path back to the loop head leaves loads
  // outstanding in the buffer the next iteration loads into.
  if (nsteps > 0) {
    for (int s = 0; s + 1 < nsteps; s += 2) {
      step(s, rka, rva, rkb, rvb);
      step(s + 1, rkb, rvb, rka, rva);
    }
    if (nsteps & 1) step(nsteps - 1, rka, rva, rkb, rvb);
  }

  // dQ = scale * acc; lane: query 16j + l16, d = 16b + 4g + r.
  void *dq = static_cast<char *>(a.dq) + plane * D * (a.f32_out ? 4 : 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ql = qloc0 + 16 * j + l16;
    if (PARTIAL && !exists(a.kmask, it.tile, ql, a.V)) continue;   // no such query
    const int row = qbase + off_l[ql];
    STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 3);
#pragma unroll
    for (int b = 0; b < DB; ++b) store4(dq, (size_t)row * D + 16 * b + 4 * g, acc[b][j] * a.scale, a.f32_out);
  }
}

// ---------------------------------------------------------------------------
// dK/dV: keys resident, query blocks streamed, each 32-key group split over a
// pair of waves on one SIMD.  Holding K, V, dK and dV of 32 keys takes about
// 316 registers per wave, which leaves one wave per SIMD and nothing to
// overlap a wave's exp work with; split, each wave needs about 150:
//   wave A (waves 0..NP-1): K and dV.  Step s: S = Q K^T, P = exp(S - lse),
//     P to LDS for its partner, dV^T += dO^T P.
//   wave B (waves NP..2NP-1): V and dK, one step behind.  Step s: dP = dO
//     V^T of block s-1, P of block s-1 from LDS, dS = P (dP - delta),
//     dK^T += Q^T dS.
// A's exp work then overlaps B's MFMAs and the other way round.  Query
// blocks pass through a three-stage LDS ring (A reads block s while B reads
// block s-1 and block s+1 is written), the P exchange through a two-stage
// buffer; one barrier per step.
// ---------------------------------------------------------------------------
template <int D, int NP, bool F32IN, bool PARTIAL>
__global__ __launch_bounds__(NP * 128) void sta_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NT = NP * 128;
  constexpr int KPI = 32 * NP;
  constexpr int STR = bwd_stride(D);
  constexpr int ST = TB * STR;
  constexpr int CHUNKS = TB * D / 8;
  constexpr int CPT = (CHUNKS + NT - 1) / NT;
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "chunk split");
  static_assert(NT >= 2 * TB, "one thread per row statistic");
  constexpr int EB = F32IN ? 4 : 2;
  constexpr int DC = D / 32;
  constexpr int DB = D / 16;
  constexpr int PB = NP * 2 * 64 * 16;            // bytes of one P exchange stage

  // LDS: Q stages 0..2, dO stages 0..2, row statistics [stage][lse*log2e |
  // delta][32], P exchange stages 0/1 [pair][kb][lane] (16 B), tile-local
  // offsets, query-tile base rows (PARTIAL: then the validity word of every
  // 32-query block of the walk).
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float *stat = reinterpret_cast<float *>(smem + 6 * ST);
  char *pbuf = reinterpret_cast<char *>(stat + 3 * 2 * TB);
  int *off_l = reinterpret_cast<int *>(pbuf + 2 * PB);
  int *lb_l = off_l + a.V;
  uint32_t *mw_l = reinterpret_cast<uint32_t *>(lb_l + a.max_list);

  const int item = __builtin_amdgcn_readfirstlane(a.sched[blockIdx.x]);
  if (item < 0) return;
  STA_CHECK(a.dbg, item < a.n_items, 0);
  const Item it = decode(item, a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const bool wa = wave < NP;            // wave-uniform
  const int pair = wa ? wave : wave - NP;

  const int l0 = __builtin_amdgcn_readfirstlane(a.list_off[it.h * a.n_tiles + it.tile]);
  const int nl = __builtin_amdgcn_readfirstlane(a.list_off[it.h * a.n_tiles + it.tile + 1]) - l0;
  for (int i = tid; i < a.V; i += NT) off_l[i] = a.off[i];
  for (int i = tid; i < nl; i += NT) {
    STA_CHECK(a.dbg, (unsigned)a.list_idx[l0 + i] < (unsigned)a.n_tiles && i < a.max_list, 1);
    lb_l[i] = a.base[a.list_idx[l0 + i]];
  }
  if constexpr (PARTIAL) {
    const int words = a.V / TB;
    for (int i = tid; i < nl * words; i += NT) mw_l[i] = a.kmask[(size_t)a.list_idx[l0 + i / words] * words + i % words];
  }

  const size_t plane = (size_t)it.bh * a.N;
  const char *qg = static_cast<const char *>(a.q) + plane * D * EB;
  const char *gg = static_cast<const char *>(a.dout) + plane * D * EB;
  const float *lse = a.lse + plane, *delta = a.delta + plane;
  const int kbase = a.base[it.tile];
  const int kloc0 = it.sub * KPI + pair * 32;
  __syncthreads();

  // The pair's 32 keys as B operands (lane: key 16kb + l16): K for wave A,
  // V for wave B.
  f16x8 frag[2][DC];
  {
    const char *src = static_cast<const char *>(wa ? a.k : a.v) + plane * D * EB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = clamp_row<PARTIAL>(kbase + off_l[kloc0 + 16 * kb + l16], a.N);
      STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 2);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const Raw8<F32IN> r = load_raw<F32IN>(src + ((size_t)row * D + 32 * c + 8 * g) * EB);
        if constexpr (F32IN)
          frag[kb][c] = __builtin_bit_cast(f16x8, wa ? score_f16<true>(r) : as_f16<true>(r));
        else
          frag[kb][c] = __builtin_bit_cast(f16x8, as_f16<false>(r));
      }
    }
  }

  const int spt = a.V / TB;
  const int nsteps = nl * spt;
  Raw8<F32IN> rq[CPT], rg[CPT];
  float rs = 0.f;   // threads 0..31: lse of query tid; 32..63: delta of query tid - 32
  auto fetch = [&](int s) {
    const int tb = lb_l[s / spt], u = s % spt;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      const int row = clamp_row<PARTIAL>(tb + off_l[u * TB + c / (D / 8)], a.N);
      STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 2);
      const size_t e = (size_t)row * D + (c % (D / 8)) * 8;
      rq[i] = load_raw<F32IN>(qg + e * EB);
      rg[i] = load_raw<F32IN>(gg + e * EB);
    }
    if (tid < 2 * TB) {
      const int row = clamp_row<PARTIAL>(tb + off_l[u * TB + (tid & (TB - 1))], a.N);
      STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 2);
      rs = tid < TB ? lse[row] * kLog2e : delta[row];
      // PARTIAL: a query that does not exist gets lse = +inf, so its P (and
      // with it dS) is exp2(-inf) = 0 in both waves of every pair.
      if (PARTIAL && tid < TB && !((mw_l[s] >> tid) & 1u)) rs = INFINITY;
    }
  };
  auto stash = [&](int stage) {
    char *qs = smem + stage * ST, *gs = smem + (3 + stage) * ST;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS < NT && c >= CHUNKS) break;
      const int o = (c / (D / 8)) * STR + (c % (D / 8)) * 16;
      *reinterpret_cast<uint4 *>(qs + o) = score_f16<F32IN>(rq[i]);
      *reinterpret_cast<uint4 *>(gs + o) = as_f16<F32IN>(rg[i]);
    }
    if (tid < 2 * TB) stat[stage * 2 * TB + tid] = rs;
  };

  // dV^T (wave A) or dK^T / scale (wave B); lane: key 16kb + l16, d 16b + 4g + r.
  f32x4 acc[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) acc[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2e = a.sl2e;
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);

  if (nsteps > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  // Iteration s: wave A works on block s (s < nsteps), wave B on block s-1
  // (s >= 1).  stage(x) = x mod 3.
  int st_cur = 0;                        // stage of block s
  for (int s = 0; s <= nsteps; ++s) {
    const int st_prev = st_cur == 0 ? 2 : st_cur - 1;
    const int st_next = st_cur == 2 ? 0 : st_cur + 1;
    const bool more = s + 1 < nsteps;
    if (more) fetch(s + 1);
    const bool active = wa ? s < nsteps : s >= 1;
    if (active) {
      const int stg = wa ? st_cur : st_prev;
      const char *qs = smem + stg * ST, *gs = smem + (3 + stg) * ST;
      const float *ls = stat + stg * 2 * TB;
      char *pex = pbuf + ((wa ? s : s - 1) & 1) * PB + pair * 2 * 64 * 16 + lane * 16;
      // A: S = Q K^T; B: dP = dO V^T.  Lane: key 16kb + l16, queries 16j + 4g + r.
      const char *rows = wa ? qs : gs;
      f32x4 t[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) t[j][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const f16x8 x = lds_f16x8(rows + (j * 16 + l16) * STR + (32 * c + 8 * g) * 2);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            t[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, frag[kb][c], t[j][kb], 0, 0, 0);
        }
      // Slots 4j + r of each 16-key block: queries 16j + 4g + r.
      f16x8 w[2];
      if (wa) {
        // P = exp2(S scale log2(e) - lse log2(e)), to registers and LDS.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 L = *reinterpret_cast<const f32x4 *>(ls + 16 * j + 4 * g);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              w[kb][4 * j + r] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(t[j][kb][r], sl2e, -L[r]));
        }
        *reinterpret_cast<f16x8 *>(pex) = w[0];
        *reinterpret_cast<f16x8 *>(pex + 64 * 16) = w[1];
      } else {
        // dS = P (dP - delta), P from the partner.
        const f16x8 p0 = *reinterpret_cast<const f16x8 *>(pex);
        const f16x8 p1 = *reinterpret_cast<const f16x8 *>(pex + 64 * 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 Dl = *reinterpret_cast<const f32x4 *>(ls + TB + 16 * j + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            w[0][4 * j + r] = (_Float16)((float)p0[4 * j + r] * (t[j][0][r] - Dl[r]));
            w[1][4 * j + r] = (_Float16)((float)p1[4 * j + r] * (t[j][1][r] - Dl[r]));
          }
        }
      }
      // A: dV^T += dO^T P; B: dK^T += Q^T dS.
      const char *tsrc = wa ? gs : qs;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const f16x8 x = lds_tr(tsrc, STR, 16 * b, trow, tcol);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, w[kb], acc[b][kb], 0, 0, 0);
      }
    }
    if (more) stash(st_next);
    __syncthreads();
    st_cur = st_next;
  }

  // dV = acc (wave A), dK = scale * acc (wave B).
  const size_t gb = plane * D * (a.f32_out ? 4 : 2);
  void *dst = static_cast<char *>(wa ? a.dv : a.dk) + gb;
  const float mul = wa ? 1.f : a.scale;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kl = kloc0 + 16 * kb + l16;
    if (PARTIAL && !exists(a.kmask, it.tile, kl, a.V)) continue;   // no such key
    const int row = kbase + off_l[kl];
    STA_CHECK(a.dbg, (unsigned)row < (unsigned)a.N, 3);
#pragma unroll
    for (int b = 0; b < DB; ++b) store4(dst, (size_t)row * D + 16 * b + 4 * g, acc[b][kb] * mul, a.f32_out);
  }
}

template <typename K>
hipError_t launch_lds(K kern, int blocks, int threads, size_t lds, const BwdArgs &a, hipStream_t s) {
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), lds, s, a);
  return hipGetLastError();
}

// PARTIAL adds the walk's validity words (one per 32-token block).
template <int D, int NW>
hipError_t dq_one(const BwdArgs &a, bool f32_in, hipStream_t s) {
  const bool part = a.kmask != nullptr;
  const size_t lds = (size_t)4 * TB * bwd_stride(D) + 4 * (a.V + a.max_list) +
                     (part ? (size_t)4 * a.max_list * (a.V / TB) : 0);
  if (part) {
    if (f32_in) return launch_lds(sta_bwd_dq_kernel<D, NW, true, true>, a.n_blocks, NW * 64, lds, a, s);
    return launch_lds(sta_bwd_dq_kernel<D, NW, false, true>, a.n_blocks, NW * 64, lds, a, s);
  }
  if (f32_in) return launch_lds(sta_bwd_dq_kernel<D, NW, true, false>, a.n_blocks, NW * 64, lds, a, s);
  return launch_lds(sta_bwd_dq_kernel<D, NW, false, false>, a.n_blocks, NW * 64, lds, a, s);
}

template <int D, int NP>
hipError_t dkdv_one(const BwdArgs &a, bool f32_in, hipStream_t s) {
  const bool part = a.kmask != nullptr;
  const size_t lds = (size_t)6 * TB * bwd_stride(D) + 4 * 6 * TB + 2 * NP * 2 * 64 * 16 +
                     4 * (a.V + a.max_list) + (part ? (size_t)4 * a.max_list * (a.V / TB) : 0);
  if (part) {
    if (f32_in) return launch_lds(sta_bwd_dkdv_kernel<D, NP, true, true>, a.n_blocks, NP * 128, lds, a, s);
    return launch_lds(sta_bwd_dkdv_kernel<D, NP, false, true>, a.n_blocks, NP * 128, lds, a, s);
  }
  if (f32_in) return launch_lds(sta_bwd_dkdv_kernel<D, NP, true, false>, a.n_blocks, NP * 128, lds, a, s);
  return launch_lds(sta_bwd_dkdv_kernel<D, NP, false, false>, a.n_blocks, NP * 128, lds, a, s);
}

}  // namespace

hipError_t launch_bwd_delta(const void *o, const void *dout, float *delta, int64_t rows, int head_dim,
                            bool f32_o, bool f32_g, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows * (head_dim / 8) + 255) / 256;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
#define STA_DELTA(D, FO, FG) hipLaunchKernelGGL((sta_bwd_delta_kernel<D, FO, FG>), grid, dim3(256), 0, stream, o, dout, delta, rows)
  if (head_dim == 128) {
    if (f32_o) { if (f32_g) STA_DELTA(128, true, true); else STA_DELTA(128, true, false); }
    else { if (f32_g) STA_DELTA(128, false, true); else STA_DELTA(128, false, false); }
  } else {
    if (f32_o) { if (f32_g) STA_DELTA(64, true, true); else STA_DELTA(64, true, false); }
    else { if (f32_g) STA_DELTA(64, false, true); else STA_DELTA(64, false, false); }
  }
#undef STA_DELTA
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs &a, int nw, int head_dim, bool f32_in, hipStream_t stream) {
  if (a.n_blocks <= 0) return hipSuccess;
  if (head_dim == 128) return nw == 4 ? dq_one<128, 4>(a, f32_in, stream) : dq_one<128, 1>(a, f32_in, stream);
  return nw == 4 ? dq_one<64, 4>(a, f32_in, stream) : dq_one<64, 1>(a, f32_in, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs &a, int pairs, int head_dim, bool f32_in, hipStream_t stream) {
  if (a.n_blocks <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (pairs == 6) return dkdv_one<128, 6>(a, f32_in, stream);
    if (pairs == 4) return dkdv_one<128, 4>(a, f32_in, stream);
    return dkdv_one<128, 1>(a, f32_in, stream);
  }
  if (pairs == 6) return dkdv_one<64, 6>(a, f32_in, stream);
  if (pairs == 4) return dkdv_one<64, 4>(a, f32_in, stream);
  return dkdv_one<64, 1>(a, f32_in, stream);
}

}  // namespace sta
