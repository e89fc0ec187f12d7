// route_common.h -- device functions shared by the gate kernels: the canonical
// softplus, the normal CDF of the load estimator and the top-k order. Internal
// to the library.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// ---------------------------------------------------------------------------
// Canonical softplus: built only from correctly rounded fp32 +, -, *, /, fma,
// rint and ldexp so that it is the identical function on every IEEE machine.
//   softplus(z) = z for z > 20; z + log1p(exp(-|z|)) for 0 < z <= 20;
//                 log1p(exp(-|z|)) for z <= 0.
// exp(y), y <= 0: y = n ln2 + r (Cody-Waite: ln2 = head + tail, head with its
// 12 low significand bits zero so n*head is exact), e^r by the degree-7 Taylor
// polynomial in Horner form, times 2^n; 0 for y < -87.
// log1p(v), 0 <= v <= 1: 2 atanh(s) with s = v / (2 + v) and
// atanh(s) = s * sum_{j=0..8} s^(2j) / (2j + 1).
// Constants are the fp32 roundings of the exact values: log2(e); ln 2 (head
// 0x1.62ep-1 and tail fp32(ln2 - head)); 1/i! for i = 2..7; 1/(2j+1), j = 1..8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float canon_exp_nonpos(float y) {
  if (y < -87.0f) return 0.0f;
  const float n = __builtin_rintf(y * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e000p-1f, y);
  r = __builtin_fmaf(-n, 0x1.0bfbe8p-15f, r);
  float p = 0x1.a01a02p-13f;
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

__device__ __forceinline__ float canon_log1p_unit(float v) {
  const float s = v / (2.0f + v);
  const float s2 = s * s;
  float q = 0x1.e1e1e2p-5f;
  q = __builtin_fmaf(q, s2, 0x1.111112p-4f);
  q = __builtin_fmaf(q, s2, 0x1.3b13b2p-4f);
  q = __builtin_fmaf(q, s2, 0x1.745d18p-4f);
  q = __builtin_fmaf(q, s2, 0x1.c71c72p-4f);
  q = __builtin_fmaf(q, s2, 0x1.24924ap-3f);
  q = __builtin_fmaf(q, s2, 0x1.99999ap-3f);
  q = __builtin_fmaf(q, s2, 0x1.555556p-2f);
  q = __builtin_fmaf(q, s2, 1.0f);
  return (s + s) * q;
}

__device__ __forceinline__ float canon_softplus(float z) {
  if (z > 20.0f) return z;
  const float v = canon_exp_nonpos(-fabsf(z));
  const float r = canon_log1p_unit(v);
  return z > 0.0f ? z + r : r;
}

__device__ __forceinline__ float std_normal_cdf(float z) { return 0.5f * erfcf(-z * 0.70710678118654752f); }

// Order used for top-k: larger value first; equal values (-0 == +0): lower index first.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }

}  // namespace moe
