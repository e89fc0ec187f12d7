// bwd_misc.hip -- the layer backward's steps around the expert products.
//
// Method (Shazeer et al. summary page): "Fragen" -- because the top-k is taken
// before the softmax, the kept gate values have continuous derivatives and the
// gradient flows back through the gate; "Kernideen" -- the noise term gives
// smooth gradients; "Load-Balancing-Losses" -- the importance loss
// w CV(sum of gates)^2 and the load loss w CV(sum of P(x,i))^2 with
// P(x,i) = Phi((clean_i - kth_excluding(H,k,i)) / Softplus((x W_noise)_i)); the
// "Switch Transformer" page's auxiliary loss, read as E sum_e f_e P_e. The
// discrete choices (top-k sets, ranks, drops) are constants of the backward.
//
//   gather     per kept assignment (t, s): dO[slot] = g_ts dy_t (the combine's
//              adjoint) and dg_ts = <dy_t, o_slot> (fp32, fixed-order wave sum);
//              dropped assignments: dg = 0
//   loss prep  one block: dL/dImportance_e and dL/dLoad_e (d CV^2 / dv in fp64)
//              and the switch loss' d/dp_e = w E f_e / T
//   gate       one wave per token: dH through the softmax over the kept logits
//              (or the full softmax for raw gates and the switch loss), the load
//              estimator's Phi' terms (its threshold's gradient goes to the expert
//              that holds kth_excluding), H = clean + eps sigma, sigma =
//              softplus(u): du = dsigma (1 - exp(-sigma)); writes dL/dclean and
//              dL/du [T, E] fp32
//   gate wgrad dW[i][e] = sum_t x[t][i] dG[t][e] in fixed-order fp32 partial sums
//              over 1024-token chunks, then a fixed-order reduction (and the bias
//              gradient sum_t dclean[t][e])
//   dx         per token: sum of its kept rows of dXp (the dispatch's adjoint)
//              + dclean_t W_gate^T (+ du_t W_noise^T), fp32, stored once
#include "common.h"
#include "stream_io.h"
#include "route_tail.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float load_elt(const void* p, int dtype, int64_t i) {
  return dtype == 1 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// One wave per assignment a = t * k + s (4 per block).
__global__ __launch_bounds__(256) void bwd_gather_kernel(BwdMiscArgs b) {
  const int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (a >= b.T * b.k) return;
  const int32_t slot = b.slot_dest[a];
  if (slot < 0) {
    if (lane == 0) b.dg[a] = 0.0f;
    return;
  }
  const int64_t t = a / b.k;
  const float g = b.topk_gate[a];
  float dot = 0.0f;
  if (b.dtype == 1) {
    const uint4* dy = reinterpret_cast<const uint4*>(b.dy) + t * (b.d / 8);
    const uint4* o = reinterpret_cast<const uint4*>(b.o) + (int64_t)slot * (b.d / 8);
    uint4* dO = reinterpret_cast<uint4*>(b.dO) + (int64_t)slot * (b.d / 8);
    for (int c = lane; c < b.d / 8; c += 64) {
      const uint4 vy = dy[c], vo = load_nt(o + c);  // o and dO rows: streamed once
      const uint32_t wy[4] = {vy.x, vy.y, vy.z, vy.w}, wo[4] = {vo.x, vo.y, vo.z, vo.w};
      uint32_t out[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float y0 = bf16_lo(wy[q]), y1 = bf16_hi(wy[q]);
        dot = __builtin_fmaf(y0, bf16_lo(wo[q]), dot);
        dot = __builtin_fmaf(y1, bf16_hi(wo[q]), dot);
        out[q] = pack_bf16x2(g * y0, g * y1);
      }
      store_nt(dO + c, uint4{out[0], out[1], out[2], out[3]});
    }
  } else {
    const float* dy = static_cast<const float*>(b.dy) + t * b.d;
    const float* o = static_cast<const float*>(b.o) + (int64_t)slot * b.d;
    float* dO = static_cast<float*>(b.dO) + (int64_t)slot * b.d;
    for (int c = lane; c < b.d; c += 64) {
      dot = __builtin_fmaf(dy[c], o[c], dot);
      dO[c] = g * dy[c];
    }
  }
  dot = wave_sum_f32(dot);
  if (lane == 0) b.dg[a] = dot;
}

// dL/dImportance, dL/dLoad (w d CV^2 / dv, population CV) and the switch loss'
// dL/dp_e, from the route's fp64 per-expert sums. One block of 1024 threads.
__global__ __launch_bounds__(1024) void bwd_loss_prep_kernel(BwdMiscArgs b) {
  __shared__ double sh[16];
  const int e = threadIdx.x;
  const int E = b.E;
  const bool on = e < E;
  const double imp = on ? b.red[E + e] : 0.0, ld = on ? b.red[2 * E + e] : 0.0;
  const double s_imp = tail::block_sum<1024>(imp, sh), s_ld = tail::block_sum<1024>(ld, sh);
  const double mi = s_imp / E, ml = s_ld / E;
  const double vi = tail::block_sum<1024>(on ? (imp - mi) * (imp - mi) : 0.0, sh) / E;
  const double vl = tail::block_sum<1024>(on ? (ld - ml) * (ld - ml) : 0.0, sh) / E;
  if (!on) return;
  // d CV^2 / dv_e = 2 (v_e - mu) / (E mu^2) - 2 var / (E mu^3); 0 for one expert
  auto dcv2 = [&](double v, double mu, double var) {
    return E <= 1 ? 0.0 : 2.0 * (v - mu) / (E * mu * mu) - 2.0 * var / (E * mu * mu * mu);
  };
  b.dimp[e] = (float)(b.w_imp * dcv2(imp, mi, vi));
  b.dload[e] = b.noisy ? (float)(b.w_load * dcv2(ld, ml, vl)) : 0.0f;
  b.dpsw[e] = (float)(b.w_switch * (double)E * ((double)b.counts_routed[e] / ((double)b.T * b.k)) / (double)b.T);
}

// One wave per token (4 per block): lane holds experts lane + 64 q. fp64
// arithmetic: the softmax Jacobians subtract nearly equal terms when one gate
// dominates (p (dp - sum p dp)), which fp32 would leave with few correct bits.
__device__ __forceinline__ double wave_sum_f64v(double v) { return tail::wave_sum_f64(v); }

template <int Q>
__global__ __launch_bounds__(256) void bwd_gate_kernel(BwdMiscArgs b) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= b.T) return;
  const int E = b.E, k = b.k;
  const float* H = b.H + t * b.lpad;
  float h[Q];
  double p[Q], dp[Q], dH[Q];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    h[q] = e < E ? H[e] : -INFINITY;
    m = fmaxf(m, h[q]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  double z = 0.0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    p[q] = lane + 64 * q < E ? exp((double)h[q] - (double)m) : 0.0;
    z += p[q];
  }
  z = wave_sum_f64v(z);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    p[q] /= z;
    dp[q] = e < E ? (double)b.dpsw[e] : 0.0;
    dH[q] = 0.0;
  }
  // dL/dg of each slot: the combine's part plus the importance loss (all slots)
  const int32_t* idx = b.topk_idx + t * k;
  const float* gt = b.topk_gate + t * k;
  double ssum = 0.0;
  for (int s = 0; s < k; ++s) ssum += (double)gt[s] * ((double)b.dg[t * k + s] + (double)b.dimp[idx[s]]);
  for (int s = 0; s < k; ++s) {
    const int e = idx[s];
    const double dgs = (double)b.dg[t * k + s] + (double)b.dimp[e];
    const double add = b.renormalize ? (double)gt[s] * (dgs - ssum) : 0.0;
    const double addp = b.renormalize ? 0.0 : dgs;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q == e) {
        dH[q] += add;
        dp[q] += addp;
      }
  }
  // softmax Jacobian of the full probabilities (raw gates and the switch loss)
  double sp = 0.0;
#pragma unroll
  for (int q = 0; q < Q; ++q) sp += p[q] * dp[q];
  sp = wave_sum_f64v(sp);
#pragma unroll
  for (int q = 0; q < Q; ++q) dH[q] += p[q] * (dp[q] - sp);

  double dcl[Q], dsg[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) dcl[q] = dsg[q] = 0.0;
  if (b.noisy) {
    // the k-th and (k+1)-th experts (H descending, lower index first on ties)
    int o_k = -1;
    const int o_k1 = idx[k - 1];  // experts at positions k and k-1 of the order
    bool in_top[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) in_top[q] = false;
    for (int s = 0; s < k; ++s)
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (lane + 64 * q == idx[s]) in_top[q] = true;
    if (k < E) {  // arg-max over the experts outside the top k
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        if (e < E && !in_top[q] && (h[q] > bv || (h[q] == bv && e < be))) {
          bv = h[q];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      o_k = be;
    }
    const double thr_in = o_k >= 0 ? (double)H[o_k] : 0.0, thr_out = (double)H[o_k1];
    const float* CL = b.CL + t * b.lpad;
    const float* SG = b.SG + t * b.lpad;
    double c_in = 0.0, c_out = 0.0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      if (e >= E || (in_top[q] && o_k < 0)) continue;  // k = E: P = 1 for kept experts
      const double sg = SG[e];
      const double zz = ((double)CL[e] - (in_top[q] ? thr_in : thr_out)) / sg;
      const double c = (double)b.dload[e] * exp(-0.5 * zz * zz) * 0.39894228040143267794 / sg;
      dcl[q] += c;
      dsg[q] -= c * zz;
      if (in_top[q]) c_in += c; else c_out += c;
    }
    c_in = wave_sum_f64v(c_in);
    c_out = wave_sum_f64v(c_out);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      if (e == o_k) dH[q] -= c_in;
      if (e == o_k1) dH[q] -= c_out;
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    if (e >= E) continue;
    b.dclean[t * E + e] = (float)(dcl[q] + dH[q]);
    if (b.noisy) {
      const double ds = dsg[q] + (double)b.noise[t * E + e] * dH[q];
      b.du[t * E + e] = (float)(ds * (1.0 - exp(-(double)b.SG[t * b.lpad + e])));
    }
  }
}

constexpr int kWgChunk = 1024;  // tokens per partial sum of the gate weight gradient

// partial[c][i][e] = sum over tokens t of chunk c of x[t][i] G[t][e]; blocks with
// blockIdx.x == 0 also write bias partials sum_t G[t][e]. 64 x 64 outputs per
// block, 4 x 4 per thread, tokens in order.
__global__ __launch_bounds__(256) void bwd_gate_wgrad_kernel(BwdMiscArgs b, const float* __restrict__ G,
                                                             float* __restrict__ part, float* __restrict__ part_b) {
  __shared__ float sx[16][64 + 4];
  __shared__ float sg[16][64 + 4];
  const int i0 = blockIdx.x * 64, e0 = blockIdx.y * 64, c = blockIdx.z;
  const int64_t t0 = (int64_t)c * kWgChunk, t1 = min((int64_t)b.T, t0 + kWgChunk);
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  float bacc = 0.0f;
  for (int64_t tt = t0; tt < t1; tt += 16) {
    for (int q = tid; q < 16 * 64; q += 256) {
      const int r = q / 64, col = q % 64;
      const int64_t t = tt + r;
      const int i = i0 + col, e = e0 + col;
      sx[r][col] = (t < t1 && i < b.d) ? load_elt(b.x, b.dtype, t * b.d + i) : 0.0f;
      sg[r][col] = (t < t1 && e < b.E) ? G[t * b.E + e] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float xa[4], ga[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u] = sx[r][ty * 4 + u];
        ga[u] = sg[r][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fmaf(xa[u], ga[v], acc[u][v]);
    }
    if (blockIdx.x == 0 && tid < 64)
      for (int r = 0; r < 16; ++r) bacc += sg[r][tid];
    __syncthreads();
  }
  float* P = part + (int64_t)c * b.d * b.E;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty * 4 + u;
    if (i >= b.d) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = e0 + tx * 4 + v;
      if (e < b.E) P[(int64_t)i * b.E + e] = acc[u][v];
    }
  }
  if (blockIdx.x == 0 && tid < 64 && e0 + tid < b.E) part_b[(int64_t)c * b.E + e0 + tid] = bacc;
}

// out[j] = sum over chunks c (in order) of part[c][j]; j < n.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part, int nchunk, int64_t n,
                                                         float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.0f;
  for (int c = 0; c < nchunk; ++c) s += part[(int64_t)c * n + j];
  out[j] = s;
}

// dx for 16 tokens per block: dispatch adjoint (sum of the tokens' kept rows of
// dXp, slot order) + dclean W_gate^T (+ du W_noise^T). Thread: columns
// i = tid, tid + 256, ... of every token of the block.
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdMiscArgs b) {
  extern __shared__ float sgr[];  // [16][E] dclean, then [16][E] du
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int nt = (int)min((int64_t)16, b.T - t0);
  for (int q = threadIdx.x; q < 16 * b.E; q += 256) {
    const int r = q / b.E, e = q % b.E;
    sgr[q] = r < nt ? b.dclean[(t0 + r) * b.E + e] : 0.0f;
    if (b.noisy) sgr[16 * b.E + q] = r < nt ? b.du[(t0 + r) * b.E + e] : 0.0f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < b.d; i += 256) {
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int e = 0; e < b.E; ++e) {
      const float wg = load_elt(b.w_gate, b.dtype, (int64_t)i * b.E + e);
      const float wn = b.noisy ? load_elt(b.w_noise, b.dtype, (int64_t)i * b.E + e) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[r] = __builtin_fmaf(sgr[r * b.E + e], wg, acc[r]);
        if (b.noisy) acc[r] = __builtin_fmaf(sgr[16 * b.E + r * b.E + e], wn, acc[r]);
      }
    }
    for (int r = 0; r < nt; ++r) {
      const int64_t t = t0 + r;
      float v = 0.0f;
      for (int s = 0; s < b.k; ++s) {
        const int32_t slot = b.slot_dest[t * b.k + s];
        if (slot >= 0) v += load_elt(b.dxp, b.dtype, (int64_t)slot * b.d + i);
      }
      v += acc[r];
      if (b.dtype == 1) static_cast<uint16_t*>(b.dx)[t * b.d + i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
      else static_cast<float*>(b.dx)[t * b.d + i] = v;
    }
  }
}

}  // namespace
}  // namespace moe

hipError_t launch_bwd_gather(const BwdMiscArgs& b, hipStream_t s) {
  const int64_t n = b.T * b.k;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe::bwd_gather_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_bwd_gate(const BwdMiscArgs& b, hipStream_t s) {
  hipLaunchKernelGGL(moe::bwd_loss_prep_kernel, dim3(1), dim3(1024), 0, s, b);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || b.T <= 0) return err;
  const dim3 grid((unsigned)((b.T + 3) / 4)), blk(256);
  const int q = (b.E + 63) / 64;
  if (q <= 1) hipLaunchKernelGGL(moe::bwd_gate_kernel<1>, grid, blk, 0, s, b);
  else if (q <= 2) hipLaunchKernelGGL(moe::bwd_gate_kernel<2>, grid, blk, 0, s, b);
  else if (q <= 4) hipLaunchKernelGGL(moe::bwd_gate_kernel<4>, grid, blk, 0, s, b);
  else if (q <= 8) hipLaunchKernelGGL(moe::bwd_gate_kernel<8>, grid, blk, 0, s, b);
  else hipLaunchKernelGGL(moe::bwd_gate_kernel<16>, grid, blk, 0, s, b);
  return hipGetLastError();
}

int64_t bwd_gate_wgrad_chunks(int64_t T) { return (T + moe::kWgChunk - 1) / moe::kWgChunk; }

// dW[d][E] (and, with db, the bias gradient [E]) from G [T][E]; part: chunks x d x E
// floats, part_b: chunks x E floats of workspace.
hipError_t launch_bwd_gate_wgrad(const BwdMiscArgs& b, const float* G, float* dW, float* db, float* part,
                                 float* part_b, hipStream_t s) {
  const int64_t nc = bwd_gate_wgrad_chunks(b.T);
  hipError_t err;
  if (nc > 0) {
    const dim3 grid((unsigned)((b.d + 63) / 64), (unsigned)((b.E + 63) / 64), (unsigned)nc);
    hipLaunchKernelGGL(moe::bwd_gate_wgrad_kernel, grid, dim3(256), 0, s, b, G, part, part_b);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t n = (int64_t)b.d * b.E;
  hipLaunchKernelGGL(moe::bwd_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, (int)nc, n, dW);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (db) {
    hipLaunchKernelGGL(moe::bwd_reduce_kernel, dim3((unsigned)((b.E + 255) / 256)), dim3(256), 0, s, part_b, (int)nc,
                       (int64_t)b.E, db);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_bwd_dx(const BwdMiscArgs& b, hipStream_t s) {
  if (b.T <= 0) return hipSuccess;
  const size_t lds = sizeof(float) * 16 * (size_t)b.E * (b.noisy ? 2 : 1);
  hipLaunchKernelGGL(moe::bwd_dx_kernel, dim3((unsigned)((b.T + 15) / 16)), dim3(256), lds, s, b);
  return hipGetLastError();
}
