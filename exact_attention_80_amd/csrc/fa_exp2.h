// fa_exp2.h -- exponential without the exponential instruction (forward).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// 2^x without the exponential instruction ([FA4N] co-design list: part of
// the exponentials on the FMA units): x = n + f with n = round(x), f in
// [-1/2, 1/2]; 2^f from a cubic that minimises the relative error on that
// interval (largest 8.4e-5, coefficients from exp2_fit.py), then scaled by
// 2^n exactly.  x is clamped at -160 first, so a masked score (-inf) gives
// exactly 0 (2^-160 is below the smallest denormal).  8 vector operations
// against one exponential instruction; host-callable for its accuracy test.
constexpr float kExp2C0 = 9.999195933e-01f;
constexpr float kExp2C1 = 6.932621598e-01f;
constexpr float kExp2C2 = 2.427141368e-01f;
constexpr float kExp2C3 = 5.521299317e-02f;
__host__ __device__ __forceinline__ float poly_exp2(float x) {
  x = __builtin_fmaxf(x, -160.f);
  const float n = __builtin_rintf(x);
  const float f = x - n;
  float q = __builtin_fmaf(kExp2C3, f, kExp2C2);
  q = __builtin_fmaf(q, f, kExp2C1);
  q = __builtin_fmaf(q, f, kExp2C0);
  return __builtin_ldexpf(q, (int)n);
}

}  // namespace fa
