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
// the integer routing is reproducible bit-for-bit. A block holds 64 tokens, one
// per lane, and E/EPW waves; wave w owns experts [w*EPW, (w+1)*EPW). A small
// prep kernel widens W_gate (and W_noise) to fp32 once per call; inside the
// loop each weight row slice is wave-uniform, arrives by scalar loads and is the
// scalar operand of v_fmac_f32, while each lane's x row arrives by 16-byte
// vector loads (bf16 widened once per value). Each wave then keeps its top-(k+1)
// candidates and softmax statistics (max, sum of exp) per token in LDS; one wave
// merges them (candidates by value descending, expert index ascending; sums
// rescaled to the common max in wave order) into the top-k, the gates and the
// thresholds of the load estimator; every wave then reduces its experts'
// probabilities, gates, counts and load estimates over the 64 tokens with
// butterfly shuffles. Per-block partial sums go to the workspace and are reduced
// in a fixed order by route_reduce / route_aux (deterministic, no float atomics).
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
  int d, E, epad, k, kk, renormalize, nblk, nw;
  const void* x;
  const float* w32;   // [d][epad] fp32 copy of W_gate (zero columns past E)
  const float* wn32;  // [d][epad] fp32 copy of W_noise, or null
  const float* gate_bias;
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
__global__ __launch_bounds__(256) void route_prep_kernel(const Tin* __restrict__ w, float* __restrict__ w32,
                                                         int d, int E, int epad) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * epad) return;
  const int64_t j = i / epad;
  const int e = (int)(i - j * epad);
  float v = 0.0f;
  if (e < E) {
    if constexpr (sizeof(Tin) == 2) {
      v = bf16_to_f32(w[j * E + e]);
    } else {
      v = w[j * E + e];
    }
  }
  w32[i] = v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;  // identical on every lane: each butterfly step adds the same two values
}

// One block = 64 tokens (one per lane) x all experts; wave w owns experts
// [w*EPW, (w+1)*EPW). Each lane accumulates its token's logits for the wave's
// experts as fixed ascending-j fma chains: x arrives per lane (16-byte vector
// loads, unpacked once) and the fp32 weight row W[j][e0 .. e0+EPW) is
// wave-uniform, read with scalar loads and used as the scalar FMA operand.
template <typename Tin, bool NOISY, int EPW>
__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  const Tin* __restrict__ x = static_cast<const Tin*>(a.x);
  const float* __restrict__ w32 = a.w32;
  const float* __restrict__ wn32 = a.wn32;
  const int d = a.d, E = a.E, k = a.k, kk = a.kk, nw = a.nw, epad = a.epad;
  const int64_t T = a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = wave * EPW;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const bool tok_ok = t < T;
  const Tin* __restrict__ xrow = x + (tok_ok ? t : T - 1) * d;  // rows past T: computed, never stored

  float acc[EPW], accn[EPW];
#pragma unroll
  for (int c = 0; c < EPW; ++c) acc[c] = accn[c] = 0.0f;

  // x chunks are prefetched one 8-wide step ahead
  constexpr int XW = sizeof(Tin) == 2 ? 1 : 2;  // 16-byte words per 8 values
  uint4 xn[XW];
#pragma unroll
  for (int q = 0; q < XW; ++q) xn[q] = reinterpret_cast<const uint4*>(xrow)[q];
  for (int j = 0; j < d; j += 8) {
    uint4 xc[XW];
#pragma unroll
    for (int q = 0; q < XW; ++q) xc[q] = xn[q];
    if (j + 8 < d) {
#pragma unroll
      for (int q = 0; q < XW; ++q) xn[q] = reinterpret_cast<const uint4*>(xrow + j + 8)[q];
    }
    float xv[8];
    if constexpr (sizeof(Tin) == 2) {
      xv[0] = bf16_lo(xc[0].x); xv[1] = bf16_hi(xc[0].x);
      xv[2] = bf16_lo(xc[0].y); xv[3] = bf16_hi(xc[0].y);
      xv[4] = bf16_lo(xc[0].z); xv[5] = bf16_hi(xc[0].z);
      xv[6] = bf16_lo(xc[0].w); xv[7] = bf16_hi(xc[0].w);
    } else {
      xv[0] = __uint_as_float(xc[0].x); xv[1] = __uint_as_float(xc[0].y);
      xv[2] = __uint_as_float(xc[0].z); xv[3] = __uint_as_float(xc[0].w);
      xv[4] = __uint_as_float(xc[XW - 1].x); xv[5] = __uint_as_float(xc[XW - 1].y);
      xv[6] = __uint_as_float(xc[XW - 1].z); xv[7] = __uint_as_float(xc[XW - 1].w);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* __restrict__ wrow = w32 + (int64_t)(j + u) * epad + e0;
#pragma unroll
      for (int c = 0; c < EPW; ++c) acc[c] = __builtin_fmaf(xv[u], wrow[c], acc[c]);
      if constexpr (NOISY) {
        const float* __restrict__ nrow = wn32 + (int64_t)(j + u) * epad + e0;
#pragma unroll
        for (int c = 0; c < EPW; ++c) accn[c] = __builtin_fmaf(xv[u], nrow[c], accn[c]);
      }
    }
  }

  // ---- logits of this wave's experts ----------------------------------------
  float h[EPW], cl[EPW], sg[EPW];
#pragma unroll
  for (int c = 0; c < EPW; ++c) {
    const int e = e0 + c;
    const bool valid = e < E;
    float cv = acc[c];
    if (a.gate_bias && valid) cv = cv + a.gate_bias[e];
    cl[c] = cv;
    if constexpr (NOISY) {
      sg[c] = canon_softplus(accn[c]);
      h[c] = valid ? __builtin_fmaf(a.noise[(tok_ok ? t : T - 1) * E + e], sg[c], cv) : -INFINITY;
    } else {
      sg[c] = 1.0f;
      h[c] = valid ? cv : -INFINITY;
    }
    if (a.logits_out && valid && tok_ok) a.logits_out[t * E + e] = h[c];
  }

  // ---- wave-local top-kk candidates and softmax statistics -------------------
  // LDS: cand_v/cand_i [nw][kk][64], wmax/wsum [nw][64], results per token.
  float* cand_v = smem;
  int* cand_i = reinterpret_cast<int*>(smem + nw * kk * 64);
  float* wmax = smem + 2 * nw * kk * 64;
  float* wsum = wmax + nw * 64;
  float* res = wsum + nw * 64;  // [5 + 2*8][64]: m, 1/S, thr_out, thr_in, have_in, sel[8], gate[8]
  {
    uint64_t taken = 0;
    float m_w = -INFINITY;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      if (r >= kk) break;
      float best = -INFINITY;
      int bi = -1;
#pragma unroll
      for (int c = 0; c < EPW; ++c) {
        if (e0 + c < E && !((taken >> c) & 1ull) && (bi < 0 || h[c] > best)) {  // strict '>': lower index on ties
          best = h[c];
          bi = c;
        }
      }
      if (bi >= 0) taken |= 1ull << bi;
      if (r == 0) m_w = best;
      cand_v[(wave * kk + r) * 64 + lane] = best;
      cand_i[(wave * kk + r) * 64 + lane] = bi >= 0 ? e0 + bi : 0x7FFFFFFF;
    }
    float s_w = 0.0f;
#pragma unroll
    for (int c = 0; c < EPW; ++c)
      if (e0 + c < E) s_w += expf(h[c] - m_w);
    wmax[wave * 64 + lane] = m_w;
    wsum[wave * 64 + lane] = s_w;
  }
  __syncthreads();

  // ---- merge (wave 0): global top-kk, softmax, gates --------------------------
  if (wave == 0) {
    float sel_v[9];
    int sel_i[9];
    float pv = INFINITY;
    int pi = -1;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      if (r >= kk) break;
      float best = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int q = 0; q < nw * kk; ++q) {
        const float v = cand_v[q * 64 + lane];
        const int i = cand_i[q * 64 + lane];
        if (i == 0x7FFFFFFF) continue;
        if (!(v < pv || (v == pv && i > pi))) continue;  // already taken: not after the previous pick
        if (bi == 0x7FFFFFFF || better(v, i, best, bi)) {
          best = v;
          bi = i;
        }
      }
      sel_v[r] = best;
      sel_i[r] = bi;
      pv = best;
      pi = bi;
    }
    float m = -INFINITY;
    for (int w = 0; w < nw; ++w) m = fmaxf(m, wmax[w * 64 + lane]);
    float S = 0.0f;
    for (int w = 0; w < nw; ++w) {
      const float mw = wmax[w * 64 + lane];
      if (mw != -INFINITY) S += wsum[w * 64 + lane] * expf(mw - m);
    }
    float g[8];
    if (a.renormalize) {
      float den = 0.0f, num[8];
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
        g[s] = expf(sel_v[s] - m) / S;
      }
    }
    float thr_out = 0.0f, thr_in = 0.0f;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      if (r == k - 1) thr_out = sel_v[r];
      if (r == k && r < kk) thr_in = sel_v[r];
    }
    res[0 * 64 + lane] = m;
    res[1 * 64 + lane] = 1.0f / S;
    res[2 * 64 + lane] = thr_out;
    res[3 * 64 + lane] = thr_in;
    res[4 * 64 + lane] = S;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s >= k) break;
      reinterpret_cast<int*>(res)[(5 + s) * 64 + lane] = sel_i[s];
      res[(13 + s) * 64 + lane] = g[s];
      if (tok_ok) {
        a.topk_idx[t * k + s] = sel_i[s];
        a.topk_gate[t * k + s] = g[s];
      }
    }
  }
  __syncthreads();

  // ---- per-expert partial sums over the block's tokens ------------------------
  const float m = res[0 * 64 + lane];
  const float S = res[4 * 64 + lane];
  const float thr_out = res[2 * 64 + lane];
  const float thr_in = res[3 * 64 + lane];
  const bool have_in = kk > k;
  int sel[8];
  float gs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s >= k) break;
    sel[s] = reinterpret_cast<const int*>(res)[(5 + s) * 64 + lane];
    gs[s] = res[(13 + s) * 64 + lane];
  }
#pragma unroll
  for (int c = 0; c < EPW; ++c) {
    const int e = e0 + c;
    const bool valid = e < E && tok_ok;
    float p = 0.0f, imp = 0.0f, cnt = 0.0f, ld = 0.0f;
    if (valid) {
      p = expf(h[c] - m) / S;
      bool in_k = false;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k) break;
        if (sel[s] == e) {
          in_k = true;
          imp = gs[s];
        }
      }
      cnt = in_k ? 1.0f : 0.0f;
      if constexpr (NOISY) {
        ld = (in_k && !have_in) ? 1.0f : std_normal_cdf((cl[c] - (in_k ? thr_in : thr_out)) / sg[c]);
      }
    }
    p = wave_sum(p);
    imp = wave_sum(imp);
    cnt = wave_sum(cnt);
    if constexpr (NOISY) ld = wave_sum(ld);
    if (lane == c && e < E) {
      const int64_t o = (int64_t)e * a.nblk + blockIdx.x;
      a.part_prob[o] = p;
      a.part_imp[o] = imp;
      a.part_load[o] = ld;
      a.part_cnt[o] = (int32_t)cnt;
    }
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

int route_epw(int E) { return E <= 256 ? 16 : (E <= 512 ? 32 : 64); }

template <typename Tin, bool NOISY, int EPW>
hipError_t launch_route_t(const RouteArgs& ra, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((route_kernel<Tin, NOISY, EPW>), dim3(ra.nblk), dim3(64 * ra.nw), lds, s, ra);
  return hipGetLastError();
}

template <typename Tin, bool NOISY>
hipError_t launch_route_epw(int epw, const RouteArgs& ra, size_t lds, hipStream_t s) {
  if (epw == 16) return launch_route_t<Tin, NOISY, 16>(ra, lds, s);
  if (epw == 32) return launch_route_t<Tin, NOISY, 32>(ra, lds, s);
  return launch_route_t<Tin, NOISY, 64>(ra, lds, s);
}

}  // namespace
}  // namespace moe

int route_tokens_per_block(int E, bool noisy) { return 64; }

size_t route_weight_floats(int d, int E) {
  const int epw = moe::route_epw(E);
  const int epad = ((E + epw - 1) / epw) * epw;
  return (size_t)d * epad;
}

hipError_t launch_route(const RouteLaunch& a, hipStream_t s) {
  using namespace moe;
  const bool noisy = a.w_noise != nullptr;
  const int epw = route_epw(a.E);
  const int nw = (a.E + epw - 1) / epw;
  const int epad = nw * epw;
  const int nblk = (int)((a.T + 63) / 64);
  hipError_t err = hipSuccess;
  if (a.T > 0) {
    const int64_t nw32 = (int64_t)a.d * epad;
    const dim3 pg((unsigned)((nw32 + 255) / 256));
    if (a.dtype == 1) {
      hipLaunchKernelGGL(route_prep_kernel<uint16_t>, pg, dim3(256), 0, s, static_cast<const uint16_t*>(a.w_gate),
                         a.w32, a.d, a.E, epad);
      if (noisy)
        hipLaunchKernelGGL(route_prep_kernel<uint16_t>, pg, dim3(256), 0, s,
                           static_cast<const uint16_t*>(a.w_noise), a.wn32, a.d, a.E, epad);
    } else {
      hipLaunchKernelGGL(route_prep_kernel<float>, pg, dim3(256), 0, s, static_cast<const float*>(a.w_gate), a.w32,
                         a.d, a.E, epad);
      if (noisy)
        hipLaunchKernelGGL(route_prep_kernel<float>, pg, dim3(256), 0, s, static_cast<const float*>(a.w_noise),
                           a.wn32, a.d, a.E, epad);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    RouteArgs ra;
    ra.T = a.T;
    ra.d = a.d;
    ra.E = a.E;
    ra.epad = epad;
    ra.k = a.k;
    ra.kk = noisy ? (a.k + 1 < a.E ? a.k + 1 : a.E) : a.k;
    ra.renormalize = a.renormalize;
    ra.nblk = nblk;
    ra.nw = nw;
    ra.x = a.x;
    ra.w32 = a.w32;
    ra.wn32 = noisy ? a.wn32 : nullptr;
    ra.gate_bias = a.gate_bias;
    ra.noise = a.noise;
    ra.topk_idx = a.topk_idx;
    ra.topk_gate = a.topk_gate;
    ra.logits_out = a.logits_out;
    ra.part_prob = a.part_prob;
    ra.part_imp = a.part_imp;
    ra.part_load = a.part_load;
    ra.part_cnt = a.part_cnt;
    const size_t lds = sizeof(float) * ((size_t)2 * nw * ra.kk * 64 + 2 * nw * 64 + 21 * 64);
    if (a.dtype == 1) {
      err = noisy ? launch_route_epw<uint16_t, true>(epw, ra, lds, s) : launch_route_epw<uint16_t, false>(epw, ra, lds, s);
    } else {
      err = noisy ? launch_route_epw<float, true>(epw, ra, lds, s) : launch_route_epw<float, false>(epw, ra, lds, s);
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
