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
//
// The device evaluates these definitions with fewer instructions and the same
// bits:
// - exp32's scaling is one ldexp(p, k): p lies in [0.70, 1.42] and
//   floor(k/2) >= -75 wherever the result is used, so p * 2^floor(k/2) is
//   exact and the two multiplies round once, as ldexp does. The range cases
//   are selects, not branches; a NaN input gives a NaN (its payload may differ).
// - The gate's two quotients, y / (2 + y) and (1 or y) / (1 + y) with
//   y = exp32(-|x|) in [0, 1], take a reciprocal, one Newton step, the
//   quotient and one remainder correction with fused multiply-adds (Markstein's
//   form: correctly rounded when the refined reciprocal is within half an ulp),
//   with no operand scaling or special-case fixup: the denominator lies in
//   [1, 3], and below y = 2^-24 it rounds to exactly 1 or 2, where every step is
//   exact. That these quotients equal the correctly rounded ones for every x is
//   established by comparing every float32 input of softplus32 and sigmoid32
//   (and of exp32) with the CPU sequences, which divide with IEEE division.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace detgrad {
namespace dm {

constexpr float kInvLn2 = 0x1.715476p+0f;  // bits 0x3FB8AA3B
constexpr float kLn2Hi = 0x1.62e4p-1f;     // bits 0x3F317200
constexpr float kLn2Lo = 0x1.7f7d1cp-20f;  // bits 0x35BFBE8E

// Polynomial and scaling of exp32 for a finite x in [-104, 89] (other x give
// a value the callers replace).
__device__ __forceinline__ float exp32_core(float x) {
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
  return __builtin_amdgcn_ldexpf(p, static_cast<int>(kf));
}

// (a NaN x fails both range tests and keeps the core's NaN)
__device__ __forceinline__ float exp32(float x) {
  const float y = exp32_core(x);
  return x > 89.0f ? __builtin_inff() : (x < -104.0f ? 0.0f : y);
}

// exp32 of x <= 0 (or NaN), as the gate calls it: e = exp32(-|x|).
__device__ __forceinline__ float exp32_nonpos(float x) { return x < -104.0f ? 0.0f : exp32_core(x); }

// n / d for d in [1, 3] and n in [0, 1] (NaN propagates): correctly rounded for
// the gate's operands (see above).
__device__ __forceinline__ float div_unit(float n, float d) {
  const float r0 = __builtin_amdgcn_rcpf(d);
  const float r = __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
  const float q0 = n * r;
  return __builtin_fmaf(__builtin_fmaf(-d, q0, n), r, q0);
}

// 2 atanh(s) to the s^13 term, given s = y / (2 + y)
__device__ __forceinline__ float log1p32_series(float s) {
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

__device__ __forceinline__ float log1p32(float y) { return log1p32_series(y / (2.0f + y)); }

// softplus32(x) and sigmoid32(x) from one e = exp32(-|x|) (e in [0, 1]).
__device__ __forceinline__ void softplus_sigmoid(float x, float& sp, float& sg) {
  const float e = exp32_nonpos(__uint_as_float(__float_as_uint(x) | 0x80000000u));
  const float m = __builtin_fmaxf(x, 0.0f);
  const float small = m + log1p32_series(div_unit(e, 2.0f + e));
  sp = x > 20.0f ? x : small;
  sg = div_unit(x >= 0.0f ? 1.0f : e, 1.0f + e);
}

}  // namespace dm
}  // namespace detgrad
