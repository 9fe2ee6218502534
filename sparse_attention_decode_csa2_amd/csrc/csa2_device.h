// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// D = A(16x32) * B(32x16) + C, fp32 accumulate.  Lane l supplies row (l % 16)
// of A and column (l % 16) of B, each with the 8 k-elements of k-group (l / 16);
// lane l receives D[4 * (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Value of the non-negative finite E4M3 (OCP E4M3FN) code c in [0, 126].
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  // subnormal: m * 2^-9 ; normal: (8 + m) * 2^(e - 10) = 1.m * 2^(e - 7)
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Value of any E4M3FN byte (sign bit honoured, 0x7F / 0xFF -> NaN).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  const float v = mag == 0x7Fu ? __uint_as_float(0x7FC00000u) : e4m3_value(mag);
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// Largest-magnitude bf16 in 16 values -> the E4M3 block scale code: the E4M3
// value nearest to amax / 6, ties to the even code, saturating at 0x7E.
// No division: with T(c) = 3 * (v(c) + v(c + 1)) = 6 * midpoint(c, c + 1)
// (exact in fp32, <= 8 significant bits), the code is the number of c in
// [0, 125] with amax > T(c), or amax == T(c) and c odd (a tie rounds up to
// the even neighbour).  That count is monotone in c, so a 7-step binary
// search finds it.
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax) {
  uint32_t lo = 0, hi = 126;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    if (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      const float T = 3.0f * (e4m3_value(mid) + e4m3_value(mid + 1));
      const bool pass = (amax > T) || (amax == T && (mid & 1u));
      lo = pass ? mid + 1 : lo;
      hi = pass ? hi : mid;
    }
  }
  return lo;
}

// The same scale code from an estimate and one exact correction: the E4M3
// code nearest to the float32 product amax * (1/6) (relative error below
// 2^-24, so its nearest code is within one of the exact one: subnormal codes
// m * 2^-9 by rounding t * 512, normal codes by rounding t's mantissa to
// three bits), then one step up or down decided by the exact thresholds T(c)
// of e4m3_scale_code (the code is the number of c with amax > T(c), or
// amax == T(c) and c odd, and that count is monotone in c).
__device__ __forceinline__ bool e4m3_scale_above(float amax, uint32_t c) {
  const float T = 3.0f * (e4m3_value(c) + e4m3_value(c + 1));
  return (amax > T) || (amax == T && (c & 1u));
}
__device__ __forceinline__ uint32_t e4m3_scale_code_fast(float amax) {
  const float t = amax * (1.0f / 6.0f);
  uint32_t c;
  if (!(t < 448.0f)) {
    c = 126u;                                   // saturated (also +inf / NaN: unspecified codes)
  } else if (t < 0x1p-6f) {
    c = (uint32_t)__builtin_rintf(t * 512.0f);  // subnormal codes 0..7 (8: the smallest normal)
  } else {
    const uint32_t u = __float_as_uint(t);
    const uint32_t e = (u >> 23) - 120u;        // E4M3 exponent field: binary exponent + 7
    c = (e << 3) | ((u >> 20) & 7u);
    c += (u & 0xFFFFFu) >= 0x80000u ? 1u : 0u;  // nearest (a carry moves to the next binade)
    c = c < 126u ? c : 126u;
  }
  if (c < 126u && e4m3_scale_above(amax, c)) return c + 1u;
  if (c > 0u && !e4m3_scale_above(amax, c - 1u)) return c - 1u;
  return c;
}

// E2M1 magnitude code (0..7) of |x| for block scale sigma > 0: nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6} * sigma, ties to the even code, saturating.
// Midpoints mu = {.25, .75, 1.25, 1.75, 2.5, 3.5, 5}; mu * sigma is exact in
// fp32 (<= 7 significant bits).  A tie at mu_i goes up exactly when the lower
// neighbour i is odd, i.e. for i in {1, 3, 5}: those thresholds use >=.
__device__ __forceinline__ uint32_t e2m1_mag_code(float ax, float s) {
  uint32_t k = 0;
  k += ax > 0.25f * s;
  k += ax >= 0.75f * s;
  k += ax > 1.25f * s;
  k += ax >= 1.75f * s;
  k += ax > 2.5f * s;
  k += ax >= 3.5f * s;
  k += ax > 5.0f * s;
  return k;
}

// Order-preserving 32-bit key of an fp32 score (larger score -> larger key),
// with -0.0 folded onto +0.0 and every NaN mapped to 1 (below -inf, whose key
// is 0x007FFFFF).  Key 0 is reserved for "no candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 1u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  if (k == 1u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace csa2
