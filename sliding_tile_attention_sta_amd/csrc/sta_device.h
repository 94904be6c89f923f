// Device helpers shared by the forward kernels: vector types and the staging
// of 8-element chunks of Q, K and V from global memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// Lazy rescaling of the online softmax: the running reference max only moves
// when a block's max exceeds it by more than 2^kTau in exp2 units, so
// probabilities stay <= 2^kTau (comfortably inside fp16) and O is rarely
// rescaled.
constexpr float kTau = 8.f;

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

// As fp16 for the P.V product.  bf16 values inside the fp16 range convert
// exactly; fp32 inputs are rounded to nearest even.  The caller keeps V within
// the fp16 range (|v| <= 65504); a saturating clamp here sits on the step's
// critical path and costs about 3 % on MI355X.
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

}  // namespace sta
