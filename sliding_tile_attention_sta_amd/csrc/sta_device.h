// Device helpers shared by the forward kernels: vector types and the staging
// of 8-element chunks of Q, K and V from global memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

// Debug builds (-DSTA_DEBUG, libsta_debug.so): bounds checks on work item
// codes, table entries, token rows and buffer offsets.  A failed check sets
// a bit in a device word (read back by sta_debug_flags) instead of
// trapping, so that a test reports it without faulting the GPU.  Bits:
// 0 work item or piece, 1 tile-list entry, 2 row or offset of a load,
// 3 row of a store, 4 LDS table index.  Release builds compile the checks
// away.
#ifdef STA_DEBUG
#define STA_CHECK(dbg, cond, bit)                                   \
  do {                                                              \
    if (!(cond)) __hip_atomic_fetch_or((dbg), 1u << (bit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
  } while (0)
#else
#define STA_CHECK(dbg, cond, bit) ((void)0)
#endif

namespace sta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// Raw global data of one 8-element chunk (converted when written to LDS, so
// that the global loads of the next step stay in flight during the math).
template <bool F32> struct Raw8;
template <> struct Raw8<false> { uint4 x; };
template <> struct Raw8<true> { float4 x, y; };

template <bool F32>
__device__ __forceinline__ Raw8<F32> load_raw(const char *p) {
  Raw8<F32> r;
  if constexpr (F32) {
    r.x = reinterpret_cast<const float4 *>(p)[0];
    r.y = reinterpret_cast<const float4 *>(p)[1];
  } else {
    r.x = *reinterpret_cast<const uint4 *>(p);
  }
  return r;
}

// As bf16 (fp32 inputs rounded to nearest even).
template <bool F32>
__device__ __forceinline__ uint4 as_bf16(const Raw8<F32> &r) {
  if constexpr (F32) {
    bf16x8 b;
    b[0] = (__bf16)r.x.x; b[1] = (__bf16)r.x.y; b[2] = (__bf16)r.x.z; b[3] = (__bf16)r.x.w;
    b[4] = (__bf16)r.y.x; b[5] = (__bf16)r.y.y; b[6] = (__bf16)r.y.z; b[7] = (__bf16)r.y.w;
    return __builtin_bit_cast(uint4, b);
  } else {
    return r.x;
  }
}

// As fp16 for the P.V product: fp32 inputs, and bf16 values below fp16's
// normal range (|v| < 2^-14, kept with fewer bits or flushed), are rounded
// to nearest even; other bf16 values inside the fp16 range convert exactly.
// Larger magnitudes (|v| > 65504) become infinities: the forward kernel
// detects those from its output and redoes the work with V scaled
// (as_f16_scaled).
template <bool F32>
__device__ __forceinline__ uint4 as_f16(const Raw8<F32> &r) {
  f16x8 h;
  if constexpr (F32) {
    h[0] = (_Float16)(r.x.x); h[1] = (_Float16)(r.x.y);
    h[2] = (_Float16)(r.x.z); h[3] = (_Float16)(r.x.w);
    h[4] = (_Float16)(r.y.x); h[5] = (_Float16)(r.y.y);
    h[6] = (_Float16)(r.y.z); h[7] = (_Float16)(r.y.w);
  } else {
    const bf16x8 b = __builtin_bit_cast(bf16x8, r.x);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)((float)b[i]);
  }
  return __builtin_bit_cast(uint4, h);
}

// As as_f16, after multiplying by a power of two (exact unless the product
// leaves fp32's normal range).
template <bool F32>
__device__ __forceinline__ uint4 as_f16_scaled(const Raw8<F32> &r, float scale) {
  f16x8 h;
  if constexpr (F32) {
    h[0] = (_Float16)(r.x.x * scale); h[1] = (_Float16)(r.x.y * scale);
    h[2] = (_Float16)(r.x.z * scale); h[3] = (_Float16)(r.x.w * scale);
    h[4] = (_Float16)(r.y.x * scale); h[5] = (_Float16)(r.y.y * scale);
    h[6] = (_Float16)(r.y.z * scale); h[7] = (_Float16)(r.y.w * scale);
  } else {
    const bf16x8 b = __builtin_bit_cast(bf16x8, r.x);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)((float)b[i] * scale);
  }
  return __builtin_bit_cast(uint4, h);
}

// Largest magnitude of the 8 elements.
template <bool F32>
__device__ __forceinline__ float max_abs8(const Raw8<F32> &r) {
  if constexpr (F32) {
    return fmaxf(fmaxf(fmaxf(fabsf(r.x.x), fabsf(r.x.y)), fmaxf(fabsf(r.x.z), fabsf(r.x.w))),
                 fmaxf(fmaxf(fabsf(r.y.x), fabsf(r.y.y)), fmaxf(fabsf(r.y.z), fabsf(r.y.w))));
  } else {
    const bf16x8 b = __builtin_bit_cast(bf16x8, r.x);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)b[i]));
    return m;
  }
}

}  // namespace sta
