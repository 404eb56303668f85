// Device helpers shared by the HIP sources of libprkv.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace prkv_dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The value lane (lane ^ M) holds, for M a power of two below 64, without a
// trip through LDS: xor 1 and 2 are DPP quad permutations, xor 4 is the
// quad reversal (xor 3) followed by the half-row mirror (xor 7), xor 8 is
// the row rotation by 8; xor 16 and xor 32 use the permlane swaps, which
// exchange the odd 16-lane rows (upper 32 lanes) of their first operand with
// the even rows (lower 32 lanes) of their second, so with both operands x a
// lane finds its partner's value in the first result if its own bit is set,
// else in the second.  Every lane of the wave must be active.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(int(x), 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(int(x), 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int y = __builtin_amdgcn_mov_dpp(int(x), 0x1B, 0xF, 0xF, true);  // quad_perm [3,2,1,0]
    return __builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, true);  // row_half_mirror
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_mov_dpp(int(x), 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}

// Inclusive prefix sums over the 64 lanes of a wave in the VALU (every lane
// active): within each 16-lane row by DPP row shifts of 1, 2, 4 and 8
// (lanes shifted in from outside the row read 0), then the last lane of row
// 0 and of row 2 added to rows 1 and 3 (row broadcast 15) and the last lane
// of row 1 to rows 2 and 3 (row broadcast 31); rows left out of a step by
// its row mask add 0.
template <int CTRL, int ROW_MASK, bool ZERO_OUTSIDE>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
  return __builtin_amdgcn_update_dpp(0u, x, CTRL, ROW_MASK, 0xF, ZERO_OUTSIDE);
}

__device__ __forceinline__ int32_t wave_scan_incl(int32_t x) {
  uint32_t v = uint32_t(x);
  v += dpp_move<0x111, 0xF, true>(v);    // row_shr:1
  v += dpp_move<0x112, 0xF, true>(v);    // row_shr:2
  v += dpp_move<0x114, 0xF, true>(v);    // row_shr:4
  v += dpp_move<0x118, 0xF, true>(v);    // row_shr:8
  v += dpp_move<0x142, 0xA, false>(v);   // row_bcast:15 into rows 1, 3
  v += dpp_move<0x143, 0xC, false>(v);   // row_bcast:31 into rows 2, 3
  return int32_t(v);
}

template <int CTRL, int ROW_MASK, bool ZERO_OUTSIDE>
__device__ __forceinline__ int64_t dpp_move64(int64_t x) {
  const uint64_t b = uint64_t(x);
  const uint32_t lo = dpp_move<CTRL, ROW_MASK, ZERO_OUTSIDE>(uint32_t(b));
  const uint32_t hi = dpp_move<CTRL, ROW_MASK, ZERO_OUTSIDE>(uint32_t(b >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t wave_scan_incl(int64_t x) {
  x += dpp_move64<0x111, 0xF, true>(x);
  x += dpp_move64<0x112, 0xF, true>(x);
  x += dpp_move64<0x114, 0xF, true>(x);
  x += dpp_move64<0x118, 0xF, true>(x);
  x += dpp_move64<0x142, 0xA, false>(x);
  x += dpp_move64<0x143, 0xC, false>(x);
  return x;
}

// Inclusive prefix sums within each 16-lane row of the wave (no carry
// between rows), for a caller whose values fill one row.
__device__ __forceinline__ int32_t row_scan_incl(int32_t x) {
  uint32_t v = uint32_t(x);
  v += dpp_move<0x111, 0xF, true>(v);
  v += dpp_move<0x112, 0xF, true>(v);
  v += dpp_move<0x114, 0xF, true>(v);
  v += dpp_move<0x118, 0xF, true>(v);
  return int32_t(v);
}

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
