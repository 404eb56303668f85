// Device helpers shared by the HIP sources of libprkv.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace prkv_dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float lo_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// x1 * c - x2 * s with c = ch + cl, s = sh + sl.  p and q (the products
// with the hi parts) are exact with their FMA error terms e and f; p - q is
// rounded once (exact when they nearly cancel), the small terms are summed,
// and the total is rounded once more: within about one float32 ulp of the
// exact value.
__device__ __forceinline__ float rot_first(float x1, float x2, f32x4 cs) {
  const float p = x1 * cs.x;
  const float e = __builtin_fmaf(x1, cs.x, -p);
  const float q = x2 * cs.z;
  const float f = __builtin_fmaf(x2, cs.z, -q);
  const float a = p - q;
  float t = __builtin_fmaf(x1, cs.y, e);
  t = __builtin_fmaf(-x2, cs.w, t);
  t = t - f;
  return a + t;
}

// x2 * c + x1 * s.
__device__ __forceinline__ float rot_second(float x1, float x2, f32x4 cs) {
  const float p = x2 * cs.x;
  const float e = __builtin_fmaf(x2, cs.x, -p);
  const float q = x1 * cs.z;
  const float f = __builtin_fmaf(x1, cs.z, -q);
  const float a = p + q;
  float t = __builtin_fmaf(x2, cs.y, e);
  t = __builtin_fmaf(x1, cs.w, t);
  t = t + f;
  return a + t;
}


}  // namespace prkv_dev
