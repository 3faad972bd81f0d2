// softmax_exact.h -- the arithmetic of next-token probabilities from logits,
// fixed to the bit so that every consumer (the probabilities kernel, the
// stochastic verifier reading logits) computes the same values.  For a row
// with maximum m and c = (float)(log2(e) / T):
//   t = (z - m) * c                 fp32
//   2^t = 2^n * P(f)                n = t rounded to the nearest integer
//                                   (ties to even), f = t - n (exact,
//                                   |f| <= 1/2), P the Taylor polynomial of
//                                   2^f = exp(f ln 2) to degree 7 in Horner
//                                   form with fused multiply-adds (truncation
//                                   error below 1e-8 relative); 0 for n < -125
//   mass(e) = floor(e * 2^40)       an exact integer (e <= 1)
//   p = e * inv                     inv = (float)(2^40 / S), S the exact
//                                   integer mass of the kept tokens
// ([SI] §4 "Token Verification"; range reduction plus a truncated Taylor
// series is the textbook method for exp.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttv {

constexpr double kLn2d = 0.6931471805599453;
constexpr double kLog2Ed = 1.4426950408889634;

// ln(2)^k / k!, each from the previous one by one multiplication and one
// division in double (constant-folded; IEEE double arithmetic).
constexpr double taylor_coef(int k) {
  double a = 1.0;
  for (int i = 1; i <= k; ++i) a = (a * kLn2d) / (double)i;
  return a;
}

__device__ __forceinline__ float exp2_taylor(float t) {
  constexpr float c1 = (float)taylor_coef(1), c2 = (float)taylor_coef(2);
  constexpr float c3 = (float)taylor_coef(3), c4 = (float)taylor_coef(4);
  constexpr float c5 = (float)taylor_coef(5), c6 = (float)taylor_coef(6);
  constexpr float c7 = (float)taylor_coef(7);
  const float n = __builtin_rintf(t);
  const float f = t - n;
  float p = c7;
  p = __builtin_fmaf(p, f, c6);
  p = __builtin_fmaf(p, f, c5);
  p = __builtin_fmaf(p, f, c4);
  p = __builtin_fmaf(p, f, c3);
  p = __builtin_fmaf(p, f, c2);
  p = __builtin_fmaf(p, f, c1);
  p = __builtin_fmaf(p, f, 1.0f);
  return n < -125.0f ? 0.0f : __builtin_amdgcn_ldexp(p, (int)n);
}

// floor(e * 2^40) as an exact integer-valued double (e in [0, 1]: the scale
// and the floor are exact in fp32)
__device__ __forceinline__ double mass40(float e) {
  return (double)__builtin_floorf(e * 1099511627776.0f);
}

// What a row's probabilities need besides its logits: the maximum, the
// normaliser, and the last kept token in the order (higher logit, then lower
// token id) -- a token is kept iff it ranks at or before (zthr, ithr).
struct RowStats {
  float m, inv, zthr;
  int ithr;
};

__device__ __forceinline__ bool row_keeps(const RowStats& s, float z, int v) {
  return z > s.zthr || (z == s.zthr && v <= s.ithr);
}

__device__ __forceinline__ float row_prob(const RowStats& s, float c, float z, int v) {
  return row_keeps(s, z, v) ? exp2_taylor((z - s.m) * c) * s.inv : 0.0f;
}

}  // namespace ttv
