// route_hier.hip -- the gate of a hierarchical MoE layer.
//
// Method: Shazeer et al. summary page, "Schluesselbegriffe": in a hierarchical
// MoE a primary gating network routes each input to secondary MoE groups; each
// gate is the noisy top-k gate of the "Methode" section, G = Softmax(KeepTopK(H,
// k)); "moe paper models" table 2 gives k = 2 for the hierarchical models. The
// layer is y = sum_i Gp(x)_i sum_j G_i(x)_j E_ij(x): a token's expert slots are
// (kept group r, kept expert q of that group), expert id i * b + j, gate
// Gp_i * G_i,j, so dispatch, expert FFN and combine are those of a flat layer
// with groups * b experts and k_group * k slots. Losses (unweighted): CV^2 of the
// primary importance (per group), CV^2 of the importance of the combined gates
// (per expert), CV^2 of the primary load estimate (noisy primary gate, else NaN).
//
// Design (gfx950): both gates' logits come from the canonical fp32 gate GEMM of
// route.hip (so routing is reproducible bit for bit); then
//   select  one wave per token: the primary top-(k_group + 1) by k_group + 1
//           wave arg-max rounds (H descending, index ascending), the softmax over
//           the kept groups, then per kept group the top-k of its b experts and
//           their softmax; writes the combined ids and gates and the primary order;
//   reduce  one wave per expert (and per group): counts and importance by a scan
//           of all assignments in a fixed order (fp64), and the primary load
//           estimate sum_t Phi((clean - kth_excluding) / softplus);
//   aux     one block: the three CV^2 values.
// Deterministic: no float atomics, fixed summation orders.
#include "common.h"
#include "route_tail.h"

namespace moe {
namespace {

// wave arg-max of (v, e): larger v first, then lower e
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oe = __shfl_xor(e, off);
    if (ov > v || (ov == v && oe < e)) {
      v = ov;
      e = oe;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per token. Lane holds primary groups lane + 64 q (q < QA) and, per
// kept group, that group's experts lane + 64 q (q < QB).
template <int QA, int QB>
__global__ __launch_bounds__(256) void route_hier_select_kernel(HierLaunch h) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= h.T) return;
  const int A = h.groups, B = h.per_group, KP = h.k_group, KS = h.k_expert;
  const float* Hp = h.Hp + t * h.lpad_p;
  const float* Hs = h.Hs + t * h.lpad_s;
  // primary order: KP (+1 when the load estimate needs the next one) arg-max rounds
  float hv[QA];
  bool taken[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int g = lane + 64 * q;
    hv[q] = g < A ? Hp[g] : -INFINITY;
    taken[q] = g >= A;
  }
  const int kk = h.noisy_p ? min(KP + 1, A) : KP;
  int ord[9];
  float ordv[9];
  for (int r = 0; r < kk; ++r) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int g = lane + 64 * q;
      if (!taken[q] && (hv[q] > bv || (hv[q] == bv && g < be))) {
        bv = hv[q];
        be = g;
      }
    }
    wave_argmax(bv, be);
    ord[r] = be;
    ordv[r] = bv;
#pragma unroll
    for (int q = 0; q < QA; ++q)
      if (lane + 64 * q == be) taken[q] = true;
  }
  // softmax over the kept groups (relative to the largest, which is ord[0])
  float zp = 0.0f;
  for (int r = 0; r < KP; ++r) zp += expf(ordv[r] - ordv[0]);
  if (lane == 0)
    for (int r = 0; r < kk; ++r) h.order_p[t * (KP + 1) + r] = ord[r];
  for (int r = 0; r < KP; ++r) {
    const float gp = expf(ordv[r] - ordv[0]) / zp;
    if (lane == 0) h.gate_p[t * KP + r] = gp;
    const int grp = ord[r];
    float sv[QB];
    bool st[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int j = lane + 64 * q;
      sv[q] = j < B ? Hs[grp * B + j] : -INFINITY;
      st[q] = j >= B;
    }
    int js[8];
    float jv[8];
    for (int u = 0; u < KS; ++u) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int j = lane + 64 * q;
        if (!st[q] && (sv[q] > bv || (sv[q] == bv && j < be))) {
          bv = sv[q];
          be = j;
        }
      }
      wave_argmax(bv, be);
      js[u] = be;
      jv[u] = bv;
#pragma unroll
      for (int q = 0; q < QB; ++q)
        if (lane + 64 * q == be) st[q] = true;
    }
    float zs = 0.0f;
    for (int u = 0; u < KS; ++u) zs += expf(jv[u] - jv[0]);
    if (lane == 0)
      for (int u = 0; u < KS; ++u) {
        const int64_t o = t * (int64_t)(KP * KS) + r * KS + u;
        h.topk_idx[o] = grp * B + js[u];
        h.topk_gate[o] = gp * (expf(jv[u] - jv[0]) / zs);
      }
  }
}

// Waves [0, E): expert e's count and importance over all T * K assignments;
// waves [E, E + A): group g's primary importance and load estimate. Fixed
// per-lane order, fp64, butterfly sums.
__global__ __launch_bounds__(256) void route_hier_reduce_kernel(HierLaunch h) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int E = h.groups * h.per_group, KP = h.k_group, K = KP * h.k_expert;
  if (w < E) {
    double cnt = 0.0, imp = 0.0;
    const int64_t n = h.T * K;
    for (int64_t a = lane; a < n; a += 64)
      if (h.topk_idx[a] == w) {
        cnt += 1.0;
        imp += h.topk_gate[a];
      }
    cnt = tail::wave_sum_f64(cnt);
    imp = tail::wave_sum_f64(imp);
    if (lane == 0) {
      h.counts_routed[w] = (int32_t)cnt;
      h.red[w] = imp;  // combined importance
    }
    return;
  }
  const int g = w - E;
  if (g >= h.groups) return;
  double imp = 0.0, ld = 0.0;
  for (int64_t t = lane; t < h.T; t += 64) {
    const int32_t* o = h.order_p + t * (KP + 1);
    bool kept = false;
    for (int r = 0; r < KP; ++r)
      if (o[r] == g) {
        kept = true;
        imp += h.gate_p[t * KP + r];
      }
    if (h.noisy_p) {
      double p = 1.0;  // k_group = groups: a kept group stays kept
      if (!kept || KP < h.groups) {
        const float thr = h.Hp[t * h.lpad_p + (kept ? o[KP] : o[KP - 1])];
        const float z = (h.CLp[t * h.lpad_p + g] - thr) / h.SGp[t * h.lpad_p + g];
        p = 0.5 * erfc(-(double)z * 0.70710678118654752440);
      }
      ld += p;
    }
  }
  imp = tail::wave_sum_f64(imp);
  ld = tail::wave_sum_f64(ld);
  if (lane == 0) {
    h.red[E + g] = imp;
    h.red[E + h.groups + g] = ld;
  }
}

__device__ double cv2_block(double v, bool on, int n, double* sh) {
  const double s = tail::block_sum<1024>(on ? v : 0.0, sh);
  const double mu = s / n;
  const double var = tail::block_sum<1024>(on ? (v - mu) * (v - mu) : 0.0, sh) / n;
  return n <= 1 ? 0.0 : var / (mu * mu);
}

__global__ __launch_bounds__(1024) void route_hier_aux_kernel(HierLaunch h) {
  __shared__ double sh[16];
  const int i = threadIdx.x;
  const int E = h.groups * h.per_group, A = h.groups;
  // E <= 1024 (checked on the host): one value per thread
  const double cp = cv2_block(i < A ? h.red[E + i] : 0.0, i < A, A, sh);
  const double cc = cv2_block(i < E ? h.red[i] : 0.0, i < E, E, sh);
  const double cl = h.noisy_p ? cv2_block(i < A ? h.red[E + A + i] : 0.0, i < A, A, sh) : 0.0;
  if (i == 0) {
    h.aux_out[0] = (float)cp;
    h.aux_out[1] = (float)cc;
    h.aux_out[2] = h.noisy_p ? (float)cl : __builtin_nanf("");
  }
}

}  // namespace
}  // namespace moe

hipError_t launch_route_hier(const HierLaunch& h, hipStream_t s) {
  using namespace moe;
  hipError_t err;
  if (h.T > 0) {
    const dim3 grid((unsigned)((h.T + 3) / 4)), blk(256);
    const int qa = (h.groups + 63) / 64, qb = (h.per_group + 63) / 64;
    if (qa <= 1 && qb <= 1) hipLaunchKernelGGL((route_hier_select_kernel<1, 1>), grid, blk, 0, s, h);
    else if (qa <= 1 && qb <= 4) hipLaunchKernelGGL((route_hier_select_kernel<1, 4>), grid, blk, 0, s, h);
    else if (qa <= 4 && qb <= 1) hipLaunchKernelGGL((route_hier_select_kernel<4, 1>), grid, blk, 0, s, h);
    else hipLaunchKernelGGL((route_hier_select_kernel<16, 16>), grid, blk, 0, s, h);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int waves = h.groups * h.per_group + h.groups;
  hipLaunchKernelGGL(route_hier_reduce_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, h);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (h.aux_out) {
    hipLaunchKernelGGL(route_hier_aux_kernel, dim3(1), dim3(1024), 0, s, h);
    err = hipGetLastError();
  }
  return err;
}
