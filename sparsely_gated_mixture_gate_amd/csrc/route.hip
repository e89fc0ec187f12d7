// route.hip -- gate logits, top-k, gate values, routed counts and balancing
// losses, fused in one kernel per block of tokens, plus two small reductions.
//
// Method (Shazeer et al. summary page, "Methode": Noisy Top-K Gating and
// Load-Balancing-Losses; "Switch Transformer" page: softmax over all experts,
// top-1, gate = mask * probabilities):
//   H(x)_e = (x W_g)_e [+ b_e] [+ eps_e * Softplus((x W_noise)_e)]
//   G(x)   = Softmax(KeepTopK(H, k))      (renormalize = 1)
//          = Softmax(H) at the kept experts (renormalize = 0)
//   losses: E * sum_e f_e P_e, CV^2(importance), CV^2(load).
//
// Design (gfx950): the gate GEMM is fp32 FMA in a fixed order -- each logit
// accumulates x[t,j] * W[j,e] from +0 for j ascending, one fma per term -- so
// the integer routing is reproducible bit-for-bit. A wave owns TM tokens and
// all experts (expert e = lane + 64*c lives in register c of lane e % 64).
// The TM tokens are wave-uniform, so x is read with scalar loads and feeds the
// FMA as a scalar operand; only W_g is staged in LDS (converted to fp32 once
// per block). Softmax statistics and the top-(k+1) selection are wave
// reductions over registers (butterfly shuffles; the comparison order is
// value descending, expert index ascending), so the [T,E] logits never touch
// LDS or HBM unless the caller asks for them. Per-block partial sums of the
// probabilities, gates, load estimates and counts go to the workspace and are
// reduced in a fixed order by route_reduce / route_aux (deterministic).
#include <float.h>

#include "common.h"

namespace moe {
namespace {

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

struct RouteArgs {
  int64_t T;
  int d, E, k, kk, renormalize, bk, nblk;
  const void* x;
  const void* w_gate;
  const float* gate_bias;
  const void* w_noise;
  const float* noise;
  int32_t* topk_idx;
  float* topk_gate;
  float* logits_out;
  float* part_prob;
  float* part_imp;
  float* part_load;
  int32_t* part_cnt;
};

template <typename Tin>
__device__ __forceinline__ float load_elem(const Tin* p, int64_t i) {
  if constexpr (sizeof(Tin) == 2) {
    return bf16_to_f32(p[i]);
  } else {
    return p[i];
  }
}

// Eight consecutive x values of one row (wave-uniform address, 16-byte aligned).
template <typename Tin>
__device__ __forceinline__ void load_x8(const Tin* __restrict__ row, int j, float* out) {
  if constexpr (sizeof(Tin) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + j);
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
    out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(row + j);
    const float4 b = *reinterpret_cast<const float4*>(row + j + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <typename Tin, bool NOISY, int TN, int TM>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  constexpr int EP = 64 * TN;
  extern __shared__ float smem[];
  const Tin* __restrict__ x = static_cast<const Tin*>(a.x);
  const Tin* __restrict__ wg = static_cast<const Tin*>(a.w_gate);
  const Tin* __restrict__ wn = static_cast<const Tin*>(a.w_noise);
  const int d = a.d, E = a.E, k = a.k, kk = a.kk, BK = a.bk;
  const int64_t T = a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * (4 * TM) + wave * TM;

  float* wg_s = smem;
  float* wn_s = smem + BK * EP;

  float acc[TM][TN];
  float accn[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int c = 0; c < TN; ++c) acc[i][c] = accn[i][c] = 0.0f;

  const Tin* xrow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + i < T ? t0 + i : T - 1;  // rows past T: computed, never stored
    xrow[i] = x + t * d;
  }

  // ---- gate GEMM: fixed ascending-j fma chains --------------------------------
  for (int j0 = 0; j0 < d; j0 += BK) {
    const int jn = min(BK, d - j0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < jn * EP; idx += 256) {
      const int jj = idx / EP;
      const int e = idx - jj * EP;
      const int64_t gi = (int64_t)(j0 + jj) * E + e;
      wg_s[idx] = e < E ? load_elem(wg, gi) : 0.0f;
      if constexpr (NOISY) wn_s[idx] = e < E ? load_elem(wn, gi) : 0.0f;
    }
    __syncthreads();
    for (int jj = 0; jj < jn; jj += 8) {
      float xv[TM][8];
#pragma unroll
      for (int i = 0; i < TM; ++i) load_x8(xrow[i], j0 + jj, xv[i]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float w[TN];
#pragma unroll
        for (int c = 0; c < TN; ++c) w[c] = wg_s[(jj + u) * EP + lane + 64 * c];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int c = 0; c < TN; ++c) acc[i][c] = __builtin_fmaf(xv[i][u], w[c], acc[i][c]);
        if constexpr (NOISY) {
          float wv[TN];
#pragma unroll
          for (int c = 0; c < TN; ++c) wv[c] = wn_s[(jj + u) * EP + lane + 64 * c];
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int c = 0; c < TN; ++c) accn[i][c] = __builtin_fmaf(xv[i][u], wv[c], accn[i][c]);
        }
      }
    }
  }

  // ---- per token: logits, top-(k+1), softmax, gates, partial sums -------------
  float s_prob[TN], s_imp[TN], s_load[TN], s_cnt[TN];
#pragma unroll
  for (int c = 0; c < TN; ++c) s_prob[c] = s_imp[c] = s_load[c] = s_cnt[c] = 0.0f;

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;  // wave-uniform
    float h[TN], cl[TN], sg[TN];
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      const int e = lane + 64 * c;
      const bool valid = e < E;
      float cv = acc[i][c];
      if (a.gate_bias && valid) cv = cv + a.gate_bias[e];
      cl[c] = cv;
      if constexpr (NOISY) {
        sg[c] = canon_softplus(accn[i][c]);
        h[c] = valid ? __builtin_fmaf(a.noise[t * E + e], sg[c], cv) : -INFINITY;
      } else {
        sg[c] = 1.0f;
        h[c] = valid ? cv : -INFINITY;
      }
      if (a.logits_out && valid) a.logits_out[t * E + e] = h[c];
    }

    // top-kk: kk rounds of a wave-wide arg-max over the untaken experts
    uint32_t taken = 0, taken_k = 0;
    float sel_v[9];
    int sel_e[9];
    float thr_out = 0.0f, thr_in = 0.0f;  // k-th and (k+1)-th largest H
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      if (r >= kk) break;
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int c = 0; c < TN; ++c) {
        const int e = lane + 64 * c;
        if (e < E && !((taken >> c) & 1u) && (be == 0x7FFFFFFF || better(h[c], e, bv, be))) {
          bv = h[c];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || better(ov, oe, bv, be))) {
          bv = ov;
          be = oe;
        }
      }
      sel_v[r] = bv;
      sel_e[r] = be;
      if (r == k - 1) thr_out = bv;
      if (r == k) thr_in = bv;
      if ((be & 63) == lane) {
        taken |= 1u << (be >> 6);
        if (r < k) taken_k |= 1u << (be >> 6);
      }
    }

    // softmax over all experts
    const float m = sel_v[0];
    float ex[TN];
    float zs = 0.0f;
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      ex[c] = (lane + 64 * c < E) ? expf(h[c] - m) : 0.0f;
      zs += ex[c];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) zs += __shfl_xor(zs, off);  // identical on every lane
    const float inv_z = 1.0f / zs;

    // gate values of the k kept experts (wave-uniform)
    float g[8];
    if (a.renormalize) {
      float den = 0.0f;
      float num[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k) break;
        num[s] = expf(sel_v[s] - sel_v[0]);
        den += num[s];
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k) break;
        g[s] = num[s] / den;
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k) break;
        g[s] = expf(sel_v[s] - m) / zs;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s >= k) break;
      if (lane == s) {
        a.topk_idx[t * k + s] = sel_e[s];
        a.topk_gate[t * k + s] = g[s];
      }
    }

    // partial sums for the losses
    const bool have_in = kk > k;
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      const int e = lane + 64 * c;
      if (e >= E) continue;
      s_prob[c] += ex[c] * inv_z;
      const bool in_k = (taken_k >> c) & 1u;
      if (in_k) {
        s_cnt[c] += 1.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (s >= k) break;
          if (sel_e[s] == e) s_imp[c] += g[s];
        }
      }
      if constexpr (NOISY) {
        float p;
        if (in_k && !have_in) {
          p = 1.0f;
        } else {
          p = std_normal_cdf((cl[c] - (in_k ? thr_in : thr_out)) / sg[c]);
        }
        s_load[c] += p;
      }
    }
  }

  // ---- block partials: waves combined in a fixed order ------------------------
  __syncthreads();
  float* red = smem;  // [4 quantities][4 waves][EP]
#pragma unroll
  for (int c = 0; c < TN; ++c) {
    const int e = lane + 64 * c;
    red[(0 * 4 + wave) * EP + e] = s_prob[c];
    red[(1 * 4 + wave) * EP + e] = s_imp[c];
    red[(2 * 4 + wave) * EP + e] = s_load[c];
    red[(3 * 4 + wave) * EP + e] = s_cnt[c];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float q[4];
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) s += red[(qi * 4 + w) * EP + e];
      q[qi] = s;
    }
    const int64_t o = (int64_t)e * a.nblk + blockIdx.x;
    a.part_prob[o] = q[0];
    a.part_imp[o] = q[1];
    a.part_load[o] = q[2];
    a.part_cnt[o] = (int32_t)q[3];
  }
}

// One block per expert: fixed-order sums of the per-block partials (fp64).
__global__ __launch_bounds__(256) void route_reduce_kernel(const float* __restrict__ part_prob,
                                                           const float* __restrict__ part_imp,
                                                           const float* __restrict__ part_load,
                                                           const int32_t* __restrict__ part_cnt, int nblk, int E,
                                                           int32_t* __restrict__ counts_routed,
                                                           double* __restrict__ red) {
  __shared__ double sd[3][256];
  __shared__ long long si[256];
  const int e = blockIdx.x;
  double p = 0.0, im = 0.0, ld = 0.0;
  long long cnt = 0;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    const int64_t o = (int64_t)e * nblk + b;
    p += part_prob[o];
    im += part_imp[o];
    ld += part_load[o];
    cnt += part_cnt[o];
  }
  sd[0][threadIdx.x] = p;
  sd[1][threadIdx.x] = im;
  sd[2][threadIdx.x] = ld;
  si[threadIdx.x] = cnt;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      sd[0][threadIdx.x] += sd[0][threadIdx.x + s];
      sd[1][threadIdx.x] += sd[1][threadIdx.x + s];
      sd[2][threadIdx.x] += sd[2][threadIdx.x + s];
      si[threadIdx.x] += si[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts_routed[e] = (int32_t)si[0];
    red[e] = sd[0][0];
    red[E + e] = sd[1][0];
    red[2 * E + e] = sd[2][0];
  }
}

__device__ double block_sum_256(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// One block: switch loss and the two CV^2 values from the per-expert sums.
__global__ __launch_bounds__(256) void route_aux_kernel(const int32_t* __restrict__ counts_routed,
                                                        const double* __restrict__ red, int E, int64_t T, int k,
                                                        int noisy, float* __restrict__ aux_out) {
  __shared__ double sh[256];
  double sw = 0.0, mi = 0.0, ml = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) {
    sw += ((double)counts_routed[e] / ((double)T * k)) * (red[e] / (double)T);
    mi += red[E + e];
    ml += red[2 * E + e];
  }
  sw = block_sum_256(sw, sh);
  mi = block_sum_256(mi, sh) / E;
  ml = block_sum_256(ml, sh) / E;
  double vi = 0.0, vl = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) {
    const double di = red[E + e] - mi;
    const double dl = red[2 * E + e] - ml;
    vi += di * di;
    vl += dl * dl;
  }
  vi = block_sum_256(vi, sh) / E;
  vl = block_sum_256(vl, sh) / E;
  if (threadIdx.x == 0) {
    const float nan = __builtin_nanf("");
    aux_out[0] = T > 0 ? (float)((double)E * sw) : nan;
    aux_out[1] = T > 0 ? (E > 1 ? (float)(vi / (mi * mi)) : 0.0f) : nan;
    aux_out[2] = (noisy && T > 0) ? (E > 1 ? (float)(vl / (ml * ml)) : 0.0f) : nan;
  }
}

__global__ void softplus_kernel(const float* __restrict__ z, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = canon_softplus(z[i]);
}

void route_shape(int E, bool noisy, int* tn, int* tm) {
  int t = 1;
  while (64 * t < E) t *= 2;
  int m;
  switch (t) {
    case 1: m = 8; break;
    case 2: m = 8; break;
    case 4: m = 4; break;
    case 8: m = 2; break;
    default: m = 1; break;
  }
  if (noisy && m > 1) m /= 2;
  *tn = t;
  *tm = m;
}

template <typename Tin, bool NOISY, int TN, int TM>
hipError_t launch_route_t(const RouteArgs& ra, size_t lds, hipStream_t s) {
  auto kern = route_kernel<Tin, NOISY, TN, TM>;
  hipLaunchKernelGGL(kern, dim3(ra.nblk), dim3(256), lds, s, ra);
  return hipGetLastError();
}

template <typename Tin, bool NOISY>
hipError_t dispatch_route_shape(int tn, int tm, const RouteArgs& ra, size_t lds, hipStream_t s) {
  if (tn == 1 && tm == 8) return launch_route_t<Tin, NOISY, 1, 8>(ra, lds, s);
  if (tn == 1 && tm == 4) return launch_route_t<Tin, NOISY, 1, 4>(ra, lds, s);
  if (tn == 2 && tm == 8) return launch_route_t<Tin, NOISY, 2, 8>(ra, lds, s);
  if (tn == 2 && tm == 4) return launch_route_t<Tin, NOISY, 2, 4>(ra, lds, s);
  if (tn == 4 && tm == 4) return launch_route_t<Tin, NOISY, 4, 4>(ra, lds, s);
  if (tn == 4 && tm == 2) return launch_route_t<Tin, NOISY, 4, 2>(ra, lds, s);
  if (tn == 8 && tm == 2) return launch_route_t<Tin, NOISY, 8, 2>(ra, lds, s);
  if (tn == 8 && tm == 1) return launch_route_t<Tin, NOISY, 8, 1>(ra, lds, s);
  if (tn == 16 && tm == 1) return launch_route_t<Tin, NOISY, 16, 1>(ra, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace moe

int route_tokens_per_block(int E, bool noisy) {
  int tn, tm;
  moe::route_shape(E, noisy, &tn, &tm);
  return 4 * tm;
}

hipError_t launch_route(const RouteLaunch& a, hipStream_t s) {
  using namespace moe;
  const bool noisy = a.w_noise != nullptr;
  int tn, tm;
  route_shape(a.E, noisy, &tn, &tm);
  const int ep = 64 * tn;
  const int tpb = 4 * tm;
  const int nblk = (int)((a.T + tpb - 1) / tpb);
  int bk = 16384 / (ep * (noisy ? 2 : 1));
  bk = bk > 64 ? 64 : bk;
  bk = (bk / 8) * 8;
  if (bk < 8) bk = 8;
  hipError_t err = hipSuccess;
  if (a.T > 0) {
    RouteArgs ra;
    ra.T = a.T;
    ra.d = a.d;
    ra.E = a.E;
    ra.k = a.k;
    ra.kk = noisy ? (a.k + 1 < a.E ? a.k + 1 : a.E) : a.k;
    ra.renormalize = a.renormalize;
    ra.bk = bk;
    ra.nblk = nblk;
    ra.x = a.x;
    ra.w_gate = a.w_gate;
    ra.gate_bias = a.gate_bias;
    ra.w_noise = a.w_noise;
    ra.noise = a.noise;
    ra.topk_idx = a.topk_idx;
    ra.topk_gate = a.topk_gate;
    ra.logits_out = a.logits_out;
    ra.part_prob = a.part_prob;
    ra.part_imp = a.part_imp;
    ra.part_load = a.part_load;
    ra.part_cnt = a.part_cnt;
    size_t stage = (size_t)bk * ep * (noisy ? 2 : 1);
    size_t redn = (size_t)16 * ep;
    size_t lds = 4 * (stage > redn ? stage : redn);
    if (a.dtype == 1) {
      err = noisy ? dispatch_route_shape<uint16_t, true>(tn, tm, ra, lds, s)
                  : dispatch_route_shape<uint16_t, false>(tn, tm, ra, lds, s);
    } else {
      err = noisy ? dispatch_route_shape<float, true>(tn, tm, ra, lds, s)
                  : dispatch_route_shape<float, false>(tn, tm, ra, lds, s);
    }
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(route_reduce_kernel, dim3(a.E), dim3(256), 0, s, a.part_prob, a.part_imp, a.part_load,
                     a.part_cnt, a.T > 0 ? nblk : 0, a.E, a.counts_routed, a.red);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.aux_out) {
    hipLaunchKernelGGL(route_aux_kernel, dim3(1), dim3(256), 0, s, a.counts_routed, a.red, a.E, a.T, a.k,
                       noisy ? 1 : 0, a.aux_out);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_softplus(const float* z, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe::softplus_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, out, n);
  return hipGetLastError();
}
