// noise.hip -- counter-based standard-normal noise for the noisy gate.
//
// Method: Shazeer et al. summary page, "Noisy Top-K Gating": the logits carry
// StandardNormal() * Softplus((x W_noise)_i). Drawn here as a counter-based
// stream, so any element can be produced alone, on any device, with identical
// bits: element (row, col) under a 64-bit key is
//   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
//   Easy as 1, 2, 3", SC 2011) of the counter (col, row low 32 bits, row high
//   32 bits, 0) and the key (low, high): ten rounds of two 32 x 32 -> 64-bit
//   multiplies by 0xD2511F53 and 0xCD9E8D57, xors with the key, the key bumped
//   by (0x9E3779B9, 0xBB67AE85) between rounds;
//   u1 = ((w0 >> 8) + 1) 2^-24 in (0, 1], u2 = (w1 >> 8) 2^-24 in [0, 1);
//   z = sqrt(-2 ln u1) cos(2 pi u2) (Box-Muller),
// with ln and cos built from correctly rounded fp32 +, -, *, /, fma and sqrt
// only: ln u = log1p(u - 1) for u >= 1/2, else e ln2 + log1p(m - 1) for
// u = m 2^e (the canonical log1p of the gate's softplus; ln2 as head + tail);
// cos(2 pi u) folded by symmetry to cos or sin of an angle in [0, pi/4] and
// Taylor polynomials of degree 10 / 11 in Horner form. Constants are the fp32
// roundings of 2 pi and 1/n!.
// Design: one thread per element, stores coalesced along a row.
#include "common.h"
#include "route_common.h"

namespace moe {
namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

__device__ __forceinline__ float ln_unit(float u) {  // u in [2^-24, 1]
  if (u >= 0.5f) return canon_log1p_unit(u - 1.0f);
  const uint32_t b = __float_as_uint(u);
  const int e = (int)(b >> 23) - 127;
  const float m = __uint_as_float((b & 0x7FFFFFu) | (127u << 23));
  const float lg = canon_log1p_unit(m - 1.0f);
  const float fe = (float)e;
  const float t = __builtin_fmaf(fe, 0x1.0bfbe8p-15f, lg);  // ln2 tail
  return __fmul_rn(fe, 0x1.62e000p-1f) + t;                 // ln2 head: exact product
}

__device__ __forceinline__ float cos_two_pi(float u) {  // u in [0, 1)
  const float w = u >= 0.5f ? u - 1.0f : u;
  float a = fabsf(w);
  float sign = 1.0f;
  if (a > 0.25f) {
    a = 0.5f - a;
    sign = -1.0f;
  }
  float p;
  if (a > 0.125f) {  // cos(2 pi a) = sin(2 pi (1/4 - a))
    const float y = __fmul_rn(0x1.921fb6p+2f, 0.25f - a);
    const float y2 = __fmul_rn(y, y);
    float q = 0x1.ae6456p-26f;                   // 1/11!
    q = __builtin_fmaf(q, -y2, 0x1.71de3ap-19f);  // 1/9!
    q = __builtin_fmaf(q, -y2, 0x1.a01a02p-13f);  // 1/7!
    q = __builtin_fmaf(q, -y2, 0x1.111112p-7f);   // 1/5!
    q = __builtin_fmaf(q, -y2, 0x1.555556p-3f);   // 1/3!
    q = __builtin_fmaf(q, -y2, 1.0f);
    p = __fmul_rn(y, q);
  } else {
    const float y = __fmul_rn(0x1.921fb6p+2f, a);
    const float y2 = __fmul_rn(y, y);
    float q = 0x1.27e4fcp-22f;                    // 1/10!
    q = __builtin_fmaf(q, -y2, 0x1.a01a02p-16f);  // 1/8!
    q = __builtin_fmaf(q, -y2, 0x1.6c16c2p-10f);  // 1/6!
    q = __builtin_fmaf(q, -y2, 0x1.555556p-5f);   // 1/4!
    q = __builtin_fmaf(q, -y2, 0.5f);             // 1/2!
    p = __builtin_fmaf(q, -y2, 1.0f);
  }
  return __fmul_rn(sign, p);
}

__global__ __launch_bounds__(256) void normal_noise_kernel(uint64_t seed, int64_t row0, int64_t rows, int cols,
                                                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * (int64_t)cols) return;
  const int64_t r = i / cols;
  const int c = (int)(i - r * cols);
  const uint64_t row = (uint64_t)(row0 + r);
  uint32_t c0 = (uint32_t)c, c1 = (uint32_t)row, c2 = (uint32_t)(row >> 32), c3 = 0u;
  philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
  const float u1 = __fmul_rn((float)((c0 >> 8) + 1u), 0x1p-24f);
  const float u2 = __fmul_rn((float)(c1 >> 8), 0x1p-24f);
  // correctly rounded fp32 square root: through fp64 (53 >= 2 * 24 + 2 bits, so the
  // second rounding cannot move the result); the fp32 square root of this toolchain is
  // off by one ulp in about 15% of cases on gfx950
  const float rad = (float)__dsqrt_rn((double)__fmul_rn(-2.0f, ln_unit(u1)));
  out[i] = __fmul_rn(rad, cos_two_pi(u2));
}

}  // namespace
}  // namespace moe

hipError_t launch_normal_noise(uint64_t seed, int64_t row0, int64_t rows, int cols, float* out, hipStream_t s) {
  const int64_t n = rows * (int64_t)cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe::normal_noise_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, seed, row0, rows,
                     cols, out);
  return hipGetLastError();
}
