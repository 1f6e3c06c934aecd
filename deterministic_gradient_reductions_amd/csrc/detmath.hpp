// Device exp / log1p / softplus / sigmoid as fixed sequences of correctly
// rounded binary32 operations.
//
// The gate backward needs these functions, and the only way a CPU reference
// can agree with the GPU bit for bit is for both to run the same sequence of
// IEEE operations: no hardware approximate instructions (their bits are not
// published), no fused multiply-add (this library is built with
// -ffp-contract=off), correctly rounded division (HIP's default for fp32).
//
// exp32(x): NaN -> NaN, x > 89 -> +inf, x < -104 -> +0; otherwise
//   k = rint(x * RN32(1/ln2)),  r = (x - k*LN2_HI) - k*LN2_LO
//   (LN2_HI = 0x3F317200 has 16 significant bits, so k*LN2_HI is exact),
//   p = Taylor polynomial of degree 7 in Horner form with coefficients
//   RN32(1/i!), each step one multiply then one add,
//   result = (p * 2^floor(k/2)) * 2^(k - floor(k/2)).
// log1p32(y), y >= 0: s = y/(2+y), z = s*s, q = z*(1/3 + z*(1/5 + ... + z/13))
//   evaluated innermost first with coefficients RN32(1/i), result = 2s + 2s*q
//   (log1p(y) = 2 atanh(y/(2+y)) truncated after the s^13 term).
// softplus32(x) = x for x > 20 (PyTorch's default threshold), else
//   max(x, +0) + log1p32(exp32(-|x|)).
// sigmoid32(x) = (x >= 0 ? 1 : e) / (1 + e) with e = exp32(-|x|).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace detgrad {
namespace dm {

constexpr float kInvLn2 = 0x1.715476p+0f;  // bits 0x3FB8AA3B
constexpr float kLn2Hi = 0x1.62e4p-1f;     // bits 0x3F317200
constexpr float kLn2Lo = 0x1.7f7d1cp-20f;  // bits 0x35BFBE8E

__device__ __forceinline__ float pow2i(int n) { return __uint_as_float(static_cast<uint32_t>(n + 127) << 23); }

__device__ __forceinline__ float exp32(float x) {
  if (x != x) return x;
  if (x > 89.0f) return __builtin_inff();
  if (x < -104.0f) return 0.0f;
  const float kf = __builtin_rintf(x * kInvLn2);
  const float r = (x - kf * kLn2Hi) - kf * kLn2Lo;
  float p = 1.0f / 5040.0f;
  p = p * r; p = p + 1.0f / 720.0f;
  p = p * r; p = p + 1.0f / 120.0f;
  p = p * r; p = p + 1.0f / 24.0f;
  p = p * r; p = p + 1.0f / 6.0f;
  p = p * r; p = p + 1.0f / 2.0f;
  p = p * r; p = p + 1.0f;
  p = p * r; p = p + 1.0f;
  const int k = static_cast<int>(kf);
  const int k1 = k >> 1;  // arithmetic shift: floor(k / 2)
  const int k2 = k - k1;
  return (p * pow2i(k1)) * pow2i(k2);
}

__device__ __forceinline__ float log1p32(float y) {
  const float s = y / (2.0f + y);
  const float z = s * s;
  float q = 1.0f / 13.0f;
  q = q * z; q = q + 1.0f / 11.0f;
  q = q * z; q = q + 1.0f / 9.0f;
  q = q * z; q = q + 1.0f / 7.0f;
  q = q * z; q = q + 1.0f / 5.0f;
  q = q * z; q = q + 1.0f / 3.0f;
  q = q * z;
  const float t = s + s;
  return t + t * q;
}

// softplus32(x) given e = exp32(-|x|)
__device__ __forceinline__ float softplus_e(float x, float e) {
  const float m = x > 0.0f ? x : 0.0f;
  const float small = m + log1p32(e);
  return x > 20.0f ? x : small;
}

// sigmoid32(x) given e = exp32(-|x|)
__device__ __forceinline__ float sigmoid_e(float x, float e) {
  const float num = x >= 0.0f ? 1.0f : e;
  return num / (1.0f + e);
}

__device__ __forceinline__ float neg_abs(float x) { return __uint_as_float(__float_as_uint(x) | 0x80000000u); }

}  // namespace dm
}  // namespace detgrad
