// route_tail.h -- the end of the routing step: fixed-order fp64 sums of the
// per-block partials the gate kernels write (per expert: softmax probabilities,
// gates, load estimates, routed counts) and the balancing losses from them.
// Shared by the route launch (its own kernels) and the forward path, which runs
// them inside the dispatch kernels. Internal to the library.
//
// Losses: Shazeer et al. summary page, "Load-Balancing-Losses" (importance and
// load, each w * CV(.)^2 with the weight left to the caller); Switch Transformer
// page (auxiliary loss: E times the sum over experts of the routed fraction times
// the mean router probability).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace tail {

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;  // identical on every lane: each butterfly step adds the same two values
}

// Sum over the NT threads of the block in a fixed order (butterfly inside each
// wave, then the wave totals in wave order); sh holds NT / 64 doubles.
template <int NT>
__device__ double block_sum(double v, double* sh) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += sh[w];
  __syncthreads();  // sh is reused by the next sum
  return r;
}

// One wave: expert e's sums over the nblk block partials (fixed order), written to
// counts_routed[e] and red[0 / E / 2E + e] (probabilities, gates, load estimates).
__device__ __forceinline__ void reduce_expert(int e, int lane, const float* __restrict__ part_prob,
                                              const float* __restrict__ part_imp,
                                              const float* __restrict__ part_load,
                                              const int32_t* __restrict__ part_cnt, int nblk, int E,
                                              int32_t* __restrict__ counts_routed, double* __restrict__ red) {
  double p = 0.0, im = 0.0, ld = 0.0, cnt = 0.0;
  constexpr int U = 8;  // loads of U rounds in flight together
  for (int b0 = lane; b0 < nblk; b0 += 64 * U) {
    float vp[U], vi[U], vl[U];
    int32_t vc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = b0 + 64 * u;
      const int64_t o = (int64_t)e * nblk + (b < nblk ? b : 0);
      vp[u] = part_prob[o];
      vi[u] = part_imp[o];
      vl[u] = part_load[o];
      vc[u] = part_cnt[o];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b0 + 64 * u >= nblk) break;
      p += vp[u];
      im += vi[u];
      ld += vl[u];
      cnt += vc[u];  // exact: integer-valued doubles far below 2^53
    }
  }
  p = wave_sum_f64(p);
  im = wave_sum_f64(im);
  ld = wave_sum_f64(ld);
  cnt = wave_sum_f64(cnt);
  if (lane == 0) {
    counts_routed[e] = (int32_t)cnt;
    red[e] = p;
    red[E + e] = im;
    red[2 * E + e] = ld;
  }
}

// The same from values already in registers, for E <= NT: thread e (have = e < E)
// holds counts_routed[e] and the three sums of expert e.
template <int NT>
__device__ void aux_from_values(bool have, int32_t cr, double r0, double r1, double r2, int E, int64_t T, int k,
                                int noisy, float* __restrict__ aux_out, double* sh) {
  const double sw = block_sum<NT>(have ? ((double)cr / ((double)T * k)) * (r0 / (double)T) : 0.0, sh);
  const double mi = block_sum<NT>(have ? r1 : 0.0, sh) / E;
  const double ml = block_sum<NT>(have ? r2 : 0.0, sh) / E;
  const double di = r1 - mi, dl = r2 - ml;
  const double vi = block_sum<NT>(have ? di * di : 0.0, sh) / E;
  const double vl = block_sum<NT>(have ? dl * dl : 0.0, sh) / E;
  if (threadIdx.x == 0) {
    const float nan = __builtin_nanf("");
    aux_out[0] = T > 0 ? (float)((double)E * sw) : nan;
    aux_out[1] = T > 0 ? (E > 1 ? (float)(vi / (mi * mi)) : 0.0f) : nan;
    aux_out[2] = (noisy && T > 0) ? (E > 1 ? (float)(vl / (ml * ml)) : 0.0f) : nan;
  }
}

// One block of NT threads: switch loss and the two CV^2 values from the
// per-expert sums (fixed order); sh holds NT / 64 doubles.
template <int NT>
__device__ void aux_block(const int32_t* __restrict__ counts_routed, const double* __restrict__ red, int E,
                          int64_t T, int k, int noisy, float* __restrict__ aux_out, double* sh) {
  double sw = 0.0, mi = 0.0, ml = 0.0;
  for (int e = threadIdx.x; e < E; e += NT) {
    sw += ((double)counts_routed[e] / ((double)T * k)) * (red[e] / (double)T);
    mi += red[E + e];
    ml += red[2 * E + e];
  }
  sw = block_sum<NT>(sw, sh);
  mi = block_sum<NT>(mi, sh) / E;
  ml = block_sum<NT>(ml, sh) / E;
  double vi = 0.0, vl = 0.0;
  for (int e = threadIdx.x; e < E; e += NT) {
    const double di = red[E + e] - mi;
    const double dl = red[2 * E + e] - ml;
    vi += di * di;
    vl += dl * dl;
  }
  vi = block_sum<NT>(vi, sh) / E;
  vl = block_sum<NT>(vl, sh) / E;
  if (threadIdx.x == 0) {
    const float nan = __builtin_nanf("");
    aux_out[0] = T > 0 ? (float)((double)E * sw) : nan;
    aux_out[1] = T > 0 ? (E > 1 ? (float)(vi / (mi * mi)) : 0.0f) : nan;
    aux_out[2] = (noisy && T > 0) ? (E > 1 ? (float)(vl / (ml * ml)) : 0.0f) : nan;
  }
}

}  // namespace tail
}  // namespace moe
