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
// the integer routing is reproducible bit-for-bit. Steps:
//   * route_prep widens W_gate (and W_noise) to fp32 once per call, laid out in
//     column blocks of BN (a noisy block holds BN/2 experts' gate columns and the
//     same experts' noise columns);
//   * route_logits is a register-blocked fp32 FMA GEMM: a block computes 64
//     tokens x BN columns, each thread 4 tokens x 8 columns, with both operands
//     streamed into a 4-stage LDS ring by direct-to-LDS buffer loads (x in its
//     storage type, widened once per value in registers). Its epilogue adds the
//     bias and, for the noisy gate, forms Softplus and H, writing H (and the clean
//     logits and Softplus values the load estimator needs) to the workspace;
//   * route_select holds 64 tokens: lane = token, each wave scans 64 experts for
//     its top-(k+1) candidates and softmax statistics; one wave merges them
//     (candidates by value descending, expert index ascending; sums rescaled to
//     the common max in wave order) into the top-k, the gates and the thresholds
//     of the load estimator; then lane = expert, each lane sums its expert's
//     probability, gate, count and load estimate over the 64 tokens in order.
// Per-block partial sums go to the workspace and are reduced in a fixed order by
// route_reduce / route_aux (deterministic, no float atomics).
#include <float.h>

#include "common.h"
#include "lds_dma.h"
#include "route_common.h"
#include "route_tail.h"

namespace moe {
namespace {

struct RouteArgs {
  int64_t T;
  int E, lpad, k, renormalize, nblk, epw;
  const float* H;     // [T][lpad] logits H (noisy: clean + eps * softplus)
  const float* CL;    // [T][lpad] clean logits x W_gate (+ b), noisy gate only
  const float* SG;    // [T][lpad] Softplus(x W_noise), noisy gate only
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

// fp32 gate weights in column blocks of BN: wc[j][q*BN + c]. Gate only: column
// c of block q is expert q*BN + c. Noisy: block q covers experts q*BN/2 .. +BN/2,
// columns c < BN/2 from W_gate and c >= BN/2 from W_noise. Zero past E.
template <typename Tin>
__global__ __launch_bounds__(256) void route_prep_kernel(const Tin* __restrict__ w_gate,
                                                         const Tin* __restrict__ w_noise, float* __restrict__ wc,
                                                         int d, int E, int ncol, int bn) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * ncol) return;
  const int64_t j = i / ncol;
  const int col = (int)(i - j * ncol);
  const int q = col / bn, c = col - q * bn;
  const Tin* src = w_gate;
  int e = q * bn + c;
  if (w_noise) {
    const int half = bn / 2;
    e = q * half + (c < half ? c : c - half);
    if (c >= half) src = w_noise;
  }
  float v = 0.0f;
  if (e < E) {
    if constexpr (sizeof(Tin) == 2) {
      v = bf16_to_f32(src[j * E + e]);
    } else {
      v = src[j * E + e];
    }
  }
  wc[i] = v;
}

constexpr int kLgTok = 64;    // tokens per logits block
constexpr int kLgJC = 32;     // j values per LDS stage
constexpr int kLgStages = 4;  // LDS ring depth

// Raw gate (and noise) accumulators for 64 tokens x one column block of BN:
// acc[t][c] = fma chain over j ascending of x[t][j] * wc[j][q*BN + c], from +0.
// Thread (tq, eg) of 16 x BN/8 owns tokens tq + 16 i (i < 4) and columns
// 4 eg .. +3 and BN/2 + 4 eg .. +3, so a wave's LDS reads of one weight row
// touch consecutive 16-byte chunks and its x reads 4 (8) consecutive rows,
// whose chunks are XOR-swizzled apart.
template <typename Tin, int BN>
__global__ __launch_bounds__(2 * BN) void route_logits_kernel(const Tin* __restrict__ x,
                                                              const float* __restrict__ wc, int64_t T, int d,
                                                              int E, int ncol, int lpad, int noisy,
                                                              const float* __restrict__ bias,
                                                              const float* __restrict__ noise, float* __restrict__ H,
                                                              float* __restrict__ CL, float* __restrict__ SG) {
  constexpr int NT = 2 * BN;
  constexpr int EG = BN / 8;
  constexpr int SZ = sizeof(Tin);
  constexpr int CPR = kLgJC * SZ / 16;      // 16-byte chunks of an x row per stage
  constexpr int SWM = (CPR < 8 ? CPR : 8) - 1;
  constexpr int X_CH = kLgTok * CPR;
  constexpr int WCR = BN / 4;               // 16-byte chunks of a weight row
  constexpr int W_CH = kLgJC * WCR;
  constexpr int X_LD = X_CH / NT, W_LD = W_CH / NT, LD = X_LD + W_LD;
  constexpr int STAGE_CH = X_CH + W_CH;
  static_assert(X_CH % NT == 0 && W_CH % NT == 0, "stage / thread mismatch");
  __shared__ uint4 smem[kLgStages * STAGE_CH];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eg = tid % EG, tq = tid / EG;
  const int64_t t0 = (int64_t)blockIdx.x * kLgTok;
  const int q = blockIdx.y;
  const int rows = (int)min<int64_t>(kLgTok, T - t0);
  const int nk = (d + kLgJC - 1) / kLgJC;

  // x rows past T are clamped (read, never stored); chunks past d in the last
  // stage are loaded but never read, weight rows past d load zero. The stage
  // offset goes into the per-lane offset, so the whole offset is range-checked
  // against the buffer size.
  const int32x4 rsX = buffer_rsrc(x + t0 * d, (uint32_t)rows * d * SZ);
  const int32x4 rsW = buffer_rsrc(wc + q * BN, (uint32_t)((int64_t)d * ncol - q * BN) * 4);
  int voffX[X_LD], voffW[W_LD];
#pragma unroll
  for (int i = 0; i < X_LD; ++i) {
    const int sl = tid + NT * i;
    const int r = sl / CPR, p = sl % CPR;
    voffX[i] = min(r, rows - 1) * d * SZ + (p ^ (r & SWM)) * 16;
  }
#pragma unroll
  for (int i = 0; i < W_LD; ++i) {
    const int sl = tid + NT * i;
    voffW[i] = (sl / WCR) * ncol * 4 + (sl % WCR) * 16;
  }
  const uint32_t lds0 = lds_address(&smem[0]);
  auto issue = [&](int kt) {
    const int st = kt % kLgStages;
#pragma unroll
    for (int i = 0; i < X_LD; ++i)
      load_to_lds(__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((st * STAGE_CH + i * NT + wave * 64) * 16)),
                  voffX[i] + kt * kLgJC * SZ, rsX, 0);
#pragma unroll
    for (int i = 0; i < W_LD; ++i)
      load_to_lds(
          __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((st * STAGE_CH + X_CH + i * NT + wave * 64) * 16)),
          voffW[i] + kt * kLgJC * ncol * 4, rsW, 0);
  };

  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;

  // One step = 8 j values: the thread's 4 x chunks (8 values of each token)
  // and 8 x 2 weight chunks, consumed in two halves of 4 j. The LDS reads of
  // half h+1 are issued before the fmas of half h (two register sets; at most
  // 12 reads in flight, within the lgkmcnt range).
  typedef uint4 XRegs[4][SZ / 2];
  typedef float4 WRegs[4][2];
  auto load_x = [&](int st, int step, XRegs& xr) {
    const uint4* sx = &smem[st * STAGE_CH];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tq + 16 * i;
#pragma unroll
      for (int h = 0; h < SZ / 2; ++h) xr[i][h] = sx[r * CPR + (((SZ / 2) * step + h) ^ (r & SWM))];
    }
  };
  auto load_w = [&](int st, int half, WRegs& w) {
    const float4* sw = reinterpret_cast<const float4*>(&smem[st * STAGE_CH + X_CH]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u][0] = sw[(half * 4 + u) * WCR + eg];
      w[u][1] = sw[(half * 4 + u) * WCR + EG + eg];
    }
  };
  float xv[4][8];
  auto unpack_x = [&](const XRegs& xr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SZ == 2) {
        const uint4 v = xr[i][0];
        xv[i][0] = bf16_lo(v.x); xv[i][1] = bf16_hi(v.x);
        xv[i][2] = bf16_lo(v.y); xv[i][3] = bf16_hi(v.y);
        xv[i][4] = bf16_lo(v.z); xv[i][5] = bf16_hi(v.z);
        xv[i][6] = bf16_lo(v.w); xv[i][7] = bf16_hi(v.w);
      } else {
        const uint4 v0 = xr[i][0], v1 = xr[i][SZ / 2 - 1];
        xv[i][0] = __uint_as_float(v0.x); xv[i][1] = __uint_as_float(v0.y);
        xv[i][2] = __uint_as_float(v0.z); xv[i][3] = __uint_as_float(v0.w);
        xv[i][4] = __uint_as_float(v1.x); xv[i][5] = __uint_as_float(v1.y);
        xv[i][6] = __uint_as_float(v1.z); xv[i][7] = __uint_as_float(v1.w);
      }
    }
  };
  auto fma_half = [&](int ub, const WRegs& w) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wv[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w, w[u][1].x, w[u][1].y, w[u][1].z, w[u][1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(xv[i][ub + u], wv[c], acc[i][c]);
    }
  };
  XRegs xs[2];
  WRegs ws[2];
  auto compute = [&](int st, int nsteps) {
    const int nh = 2 * nsteps;
    load_x(st, 0, xs[0]);
    load_w(st, 0, ws[0]);
#pragma unroll
    for (int h = 0; h < kLgJC / 4; ++h) {
      if (h >= nh) break;
      if (h + 1 < nh) {
        if (((h + 1) & 1) == 0) load_x(st, (h + 1) / 2, xs[((h + 1) / 2) & 1]);
        load_w(st, h + 1, ws[(h + 1) & 1]);
      }
      if ((h & 1) == 0) unpack_x(xs[(h / 2) & 1]);
      fma_half(4 * (h & 1), ws[h & 1]);
    }
  };

#pragma unroll
  for (int t = 0; t < kLgStages - 1; ++t)
    if (t < nk) issue(t);
  for (int kt = 0; kt < nk; ++kt) {
    wait_tiles<LD, kLgStages - 2>(min(kLgStages - 2, nk - 1 - kt));
    block_barrier();  // stage kt is in LDS for every wave; the buffer of stage kt-1 is free
    if (kt + kLgStages - 1 < nk) issue(kt + kLgStages - 1);
    compute(kt % kLgStages, min(kLgJC, d - kt * kLgJC) / 8);
  }

  // Epilogue: logits of the thread's 4 tokens x 4 experts (x 2 for the gate-only
  // layout). Clean logit = acc + bias (one rounding); noisy: softplus of the noise
  // accumulator and H = fma(eps, softplus, clean).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + tq + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (noisy && half == 1) break;
      const int e = noisy ? q * (BN / 2) + 4 * eg : q * BN + half * (BN / 2) + 4 * eg;
      if (e >= lpad) continue;
      float cv[4], sg[4], hv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool valid = e + c < E;
        cv[c] = acc[i][4 * half + c];
        if (bias && valid) cv[c] = cv[c] + bias[e + c];
        hv[c] = cv[c];
        if (noisy) {
          sg[c] = canon_softplus(acc[i][4 + c]);
          if (valid) hv[c] = __builtin_fmaf(noise[t * E + e + c], sg[c], cv[c]);
        }
      }
      *reinterpret_cast<float4*>(H + t * lpad + e) = float4{hv[0], hv[1], hv[2], hv[3]};
      if (noisy) {
        *reinterpret_cast<float4*>(CL + t * lpad + e) = float4{cv[0], cv[1], cv[2], cv[3]};
        *reinterpret_cast<float4*>(SG + t * lpad + e) = float4{sg[0], sg[1], sg[2], sg[3]};
      }
    }
  }
}

// Per-token routing and per-expert partial sums for a block of 64 tokens and
// 16 waves.
//  1. lane = token: wave w scans experts [w*epw, (w+1)*epw), keeping the
//     top-KK (value descending, index ascending) and the softmax statistics
//     (max, then sum of exp) of its range;
//  2. wave 0 merges the 16 sorted candidate lists (sums rescaled to the common
//     max in wave order) into the top-k, the gates and the thresholds of the
//     load estimator, and writes the token's results;
//  3. lane = expert: wave w takes expert group w % G (G = ceil(E/64)) and token
//     slice w / G of 16/G slices, accumulating each expert's softmax
//     probability, gate, count and load estimate over its slice in token order;
//     the slices are then added in slice order.
template <bool NOISY, int KK>
__global__ __launch_bounds__(1024) void route_select_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  constexpr int NW = 16;
  constexpr int KS = KK < 8 ? KK : 8;  // selectable slots (k <= KS)
  constexpr int RS = 24;  // floats per token in res: m, S, thr_out, thr_in, sel[8], gate[8], pad
  const int E = a.E, k = a.k, lpad = a.lpad, epw = a.epw;
  const int64_t T = a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int nt = (int)min<int64_t>(64, T - t0);
  float* cand_v = smem;                                        // [NW][KK][64]
  int* cand_i = reinterpret_cast<int*>(smem + NW * KK * 64);   // [NW][KK][64]
  float* wmax = smem + 2 * NW * KK * 64;                       // [NW][64]
  float* wsum = wmax + NW * 64;                                // [NW][64]
  float* res = wsum + NW * 64;                                 // [64][RS]
  float* part = res + 64 * RS;                                 // [4][NW*64]: slice partials

  // ---- 1. lane = token: candidates and softmax statistics of this wave's range
  {
    const int e_lo = min(E, wave * epw), e_hi = min(E, e_lo + epw);
    const int64_t t = t0 + lane;
    const float* hrow = a.H + (t < T ? t : T - 1) * lpad;  // rows past T: computed, never stored
    float bv[KK];
    int bi[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7FFFFFFF;
    }
    for (int e0 = e_lo; e0 < e_hi; e0 += 16) {
      float hv[16];  // all four loads in flight together
#pragma unroll
      for (int c = 0; c < 16; c += 4) {
        float4 h4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (e0 + c < e_hi) h4 = *reinterpret_cast<const float4*>(hrow + e0 + c);
        hv[c] = h4.x; hv[c + 1] = h4.y; hv[c + 2] = h4.z; hv[c + 3] = h4.w;
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        float v = hv[c];
        int i = e0 + c;
        if (i >= e_hi) break;
        if (!better(v, i, bv[KK - 1], bi[KK - 1])) continue;
#pragma unroll
        for (int r = 0; r < KK; ++r) {
          if (better(v, i, bv[r], bi[r])) {
            const float tv = bv[r];
            const int ti = bi[r];
            bv[r] = v;
            bi[r] = i;
            v = tv;
            i = ti;
          }
        }
      }
    }
    const float m_w = bv[0];
    float s_w = 0.0f;
    for (int e0 = e_lo; e0 < e_hi; e0 += 16) {
      float hv[16];
#pragma unroll
      for (int c = 0; c < 16; c += 4) {
        float4 h4 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e0 + c < e_hi) h4 = *reinterpret_cast<const float4*>(hrow + e0 + c);
        hv[c] = h4.x; hv[c + 1] = h4.y; hv[c + 2] = h4.z; hv[c + 3] = h4.w;
      }
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (e0 + c < e_hi) s_w += expf(hv[c] - m_w);
    }
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      cand_v[(wave * KK + r) * 64 + lane] = bv[r];
      cand_i[(wave * KK + r) * 64 + lane] = bi[r];
    }
    wmax[wave * 64 + lane] = e_lo < e_hi ? m_w : -INFINITY;
    wsum[wave * 64 + lane] = s_w;
  }
  __syncthreads();

  // ---- 2. merge (wave 0): global top-kk, softmax, gates --------------------------
  if (wave == 0) {
    const int64_t t = t0 + lane;
    float sel_v[KK];
    int sel_i[KK];
    uint64_t heads = 0;  // 4 bits per list: index of its next candidate
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      float best = -INFINITY;
      int bi = 0x7FFFFFFF, bw = -1;
      for (int w = 0; w < NW; ++w) {
        const int h = (int)((heads >> (4 * w)) & 15u);
        if (h >= KK) continue;
        const float v = cand_v[(w * KK + h) * 64 + lane];
        const int i = cand_i[(w * KK + h) * 64 + lane];
        if (i == 0x7FFFFFFF) continue;
        if (bw < 0 || better(v, i, best, bi)) {
          best = v;
          bi = i;
          bw = w;
        }
      }
      if (bw >= 0) heads += uint64_t(1) << (4 * bw);
      sel_v[r] = best;
      sel_i[r] = bi;
    }
    float m = -INFINITY;
    for (int w = 0; w < NW; ++w) m = fmaxf(m, wmax[w * 64 + lane]);
    float S = 0.0f;
    for (int w = 0; w < NW; ++w) {
      const float mw = wmax[w * 64 + lane];
      if (mw != -INFINITY) S += wsum[w * 64 + lane] * expf(mw - m);
    }
    float g[8];
    if (a.renormalize) {
      float den = 0.0f, num[8];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s >= k) break;
        num[s] = expf(sel_v[s] - sel_v[0]);
        den += num[s];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s >= k) break;
        g[s] = num[s] / den;
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s >= k) break;
        g[s] = expf(sel_v[s] - m) / S;
      }
    }
    float thr_out = 0.0f, thr_in = 0.0f;
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      if (r == k - 1) thr_out = sel_v[r];
      if (r == k) thr_in = sel_v[r];
    }
    float* rt = res + lane * RS;
    rt[0] = m;
    rt[1] = S;
    rt[2] = thr_out;
    rt[3] = thr_in;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s >= k) break;
      reinterpret_cast<int*>(rt)[4 + s] = sel_i[s];
      rt[12 + s] = g[s];
      if (t < T) {
        a.topk_idx[t * k + s] = sel_i[s];
        a.topk_gate[t * k + s] = g[s];
      }
    }
  }
  __syncthreads();

  // ---- 3. lane = expert: sums over a token slice, in token order ----------------
  const int G = (E + 63) / 64;
  const int TS = NW / G;
  const int TL = (64 + TS - 1) / TS;
  const int gq = wave % G, ts = wave / G;
  const int e = gq * 64 + lane;
  if (ts < TS && e < E) {
    const bool have_in = KK > k;
    const int tl_lo = min(nt, ts * TL), tl_hi = min(nt, tl_lo + TL);
    float p_sum = 0.0f, imp_sum = 0.0f, ld_sum = 0.0f;
    int cnt = 0;
    constexpr int TB = NOISY ? 8 : 16;  // tokens whose loads are in flight together
    for (int tb = tl_lo; tb < tl_hi; tb += TB) {
      float hb[TB], cb[TB], sb[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int64_t t = t0 + min(tb + u, tl_hi - 1);
        hb[u] = a.H[t * lpad + e];
        if constexpr (NOISY) {
          cb[u] = a.CL[t * lpad + e];
          sb[u] = a.SG[t * lpad + e];
        }
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int tl = tb + u;
        if (tl >= tl_hi) break;
        const float* rt = res + tl * RS;
        const float h = hb[u];
        if (a.logits_out) a.logits_out[(t0 + tl) * E + e] = h;
        p_sum += expf(h - rt[0]) / rt[1];
        bool in_k = false;
        float gk = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s >= k) break;
          if (reinterpret_cast<const int*>(rt)[4 + s] == e) {
            in_k = true;
            gk = rt[12 + s];
          }
        }
        imp_sum += gk;
        cnt += in_k ? 1 : 0;
        if constexpr (NOISY) {
          const float thr = in_k ? rt[3] : rt[2];
          ld_sum += (in_k && !have_in) ? 1.0f : std_normal_cdf((cb[u] - thr) / sb[u]);
        }
      }
    }
    const int o = ts * (G * 64) + e;
    part[0 * NW * 64 + o] = p_sum;
    part[1 * NW * 64 + o] = imp_sum;
    part[2 * NW * 64 + o] = ld_sum;
    reinterpret_cast<int*>(part)[3 * NW * 64 + o] = cnt;
  }
  __syncthreads();
  const int ef = threadIdx.x;
  if (ef < E) {
    float p_sum = 0.0f, imp_sum = 0.0f, ld_sum = 0.0f;
    int cnt = 0;
    for (int s = 0; s < TS; ++s) {
      const int o = s * (G * 64) + ef;
      p_sum += part[0 * NW * 64 + o];
      imp_sum += part[1 * NW * 64 + o];
      ld_sum += part[2 * NW * 64 + o];
      cnt += reinterpret_cast<const int*>(part)[3 * NW * 64 + o];
    }
    const int64_t o = (int64_t)ef * a.nblk + blockIdx.x;
    a.part_prob[o] = p_sum;
    a.part_imp[o] = imp_sum;
    a.part_load[o] = ld_sum;
    a.part_cnt[o] = cnt;
  }
}

constexpr int kReduceThreads = 512;  // 8 waves, one expert each

// Fixed-order sums (fp64) of the per-block partials, one expert per wave.
__global__ __launch_bounds__(kReduceThreads) void route_reduce_kernel(
    const float* __restrict__ part_prob, const float* __restrict__ part_imp, const float* __restrict__ part_load,
    const int32_t* __restrict__ part_cnt, int nblk, int E, int32_t* __restrict__ counts_routed,
    double* __restrict__ red) {
  const int e = blockIdx.x * (kReduceThreads / 64) + (threadIdx.x >> 6);
  if (e >= E) return;
  tail::reduce_expert(e, threadIdx.x & 63, part_prob, part_imp, part_load, part_cnt, nblk, E, counts_routed, red);
}

// One block: switch loss and the two CV^2 values from the per-expert sums.
__global__ __launch_bounds__(kReduceThreads) void route_aux_kernel(const int32_t* __restrict__ counts_routed,
                                                                   const double* __restrict__ red, int E, int64_t T,
                                                                   int k, int noisy, float* __restrict__ aux_out) {
  __shared__ double sh[kReduceThreads / 64];
  tail::aux_block<kReduceThreads>(counts_routed, red, E, T, k, noisy, aux_out, sh);
}

__global__ void softplus_kernel(const float* __restrict__ z, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = canon_softplus(z[i]);
}

template <bool NOISY, int KK>
hipError_t launch_select_t(const RouteArgs& ra, hipStream_t s) {
  const size_t lds = sizeof(float) * ((size_t)2 * 16 * KK * 64 + 2 * 16 * 64 + 64 * 24 + 4 * 16 * 64);
  hipLaunchKernelGGL((route_select_kernel<NOISY, KK>), dim3(ra.nblk), dim3(1024), lds, s, ra);
  return hipGetLastError();
}

template <bool NOISY>
hipError_t launch_select(int kk, const RouteArgs& ra, hipStream_t s) {
  switch (kk) {
    case 1: return launch_select_t<NOISY, 1>(ra, s);
    case 2: return launch_select_t<NOISY, 2>(ra, s);
    case 3: return launch_select_t<NOISY, 3>(ra, s);
    case 4: return launch_select_t<NOISY, 4>(ra, s);
    case 5: return launch_select_t<NOISY, 5>(ra, s);
    case 6: return launch_select_t<NOISY, 6>(ra, s);
    case 7: return launch_select_t<NOISY, 7>(ra, s);
    case 8: return launch_select_t<NOISY, 8>(ra, s);
    default: return launch_select_t<NOISY, 9>(ra, s);
  }
}

// Column block of the logits GEMM: 64 columns for small gate-only layers, else 128.
int route_bn(int E, bool noisy) { return (!noisy && E <= 64) ? 64 : 128; }
int route_ncol(int E, bool noisy) {
  const int bn = route_bn(E, noisy);
  if (noisy) return ((E + bn / 2 - 1) / (bn / 2)) * bn;
  return ((E + bn - 1) / bn) * bn;
}
int route_lpad(int E) { return (E + 3) & ~3; }

struct LogitBufs {
  float *H, *CL, *SG;
};
LogitBufs logit_bufs(const RouteLaunch& a, bool noisy) {
  const size_t n = (size_t)a.T * route_lpad(a.E);
  return LogitBufs{a.lg, noisy ? a.lg + n : nullptr, noisy ? a.lg + 2 * n : nullptr};
}

template <typename Tin>
hipError_t launch_logits(const RouteLaunch& a, bool noisy, hipStream_t s) {
  const LogitBufs lb = logit_bufs(a, noisy);
  const int bn = route_bn(a.E, noisy), ncol = route_ncol(a.E, noisy);
  const int64_t nwc = (int64_t)a.d * ncol;
  hipLaunchKernelGGL(route_prep_kernel<Tin>, dim3((unsigned)((nwc + 255) / 256)), dim3(256), 0, s,
                     static_cast<const Tin*>(a.w_gate), static_cast<const Tin*>(noisy ? a.w_noise : nullptr), a.wc,
                     a.d, a.E, ncol, bn);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)((a.T + kLgTok - 1) / kLgTok), (unsigned)(ncol / bn));
  const int lpad = route_lpad(a.E);
  if (bn == 64) {
    hipLaunchKernelGGL((route_logits_kernel<Tin, 64>), grid, dim3(128), 0, s, static_cast<const Tin*>(a.x), a.wc,
                       a.T, a.d, a.E, ncol, lpad, noisy ? 1 : 0, a.gate_bias, a.noise, lb.H, lb.CL, lb.SG);
  } else {
    hipLaunchKernelGGL((route_logits_kernel<Tin, 128>), grid, dim3(256), 0, s, static_cast<const Tin*>(a.x), a.wc,
                       a.T, a.d, a.E, ncol, lpad, noisy ? 1 : 0, a.gate_bias, a.noise, lb.H, lb.CL, lb.SG);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

int route_partial_blocks(int64_t T, int E, int dtype, int gate_mode, bool logits_out) {
  if (T <= 0) return 0;
  // gate mode 3 exports the certified gate's logits and bounds through logits_out
  const bool fused = route_fused_supported(dtype, E) && gate_mode != 1 && (!logits_out || gate_mode == 3);
  const int tpb = fused ? route_fused_tokens(T) : 64;
  return (int)((T + tpb - 1) / tpb);
}

size_t route_weight_floats(int d, int E, bool noisy) { return (size_t)d * moe::route_ncol(E, noisy); }

size_t route_logit_floats(int64_t T, int E, bool noisy) { return (size_t)T * moe::route_lpad(E) * (noisy ? 3 : 1); }

hipError_t launch_route(const RouteLaunch& a, hipStream_t s) {
  using namespace moe;
  const bool noisy = a.w_noise != nullptr;
  const int nblk = route_partial_blocks(a.T, a.E, a.dtype, a.gate_mode, a.logits_out != nullptr);
  hipError_t err = hipSuccess;
  const bool fused =
      route_fused_supported(a.dtype, a.E) && a.gate_mode != 1 && (a.logits_out == nullptr || a.gate_mode == 3);
  if (a.T > 0 && fused) {
    const LogitBufs lb = logit_bufs(a, noisy);
    err = launch_route_fused(a, noisy, a.gate_mode == 2 ? 1 : 0, lb.CL, lb.SG, route_lpad(a.E), s);
    if (err != hipSuccess) return err;
  } else if (a.T > 0) {
    err = a.dtype == 1 ? launch_logits<uint16_t>(a, noisy, s) : launch_logits<float>(a, noisy, s);
    if (err != hipSuccess) return err;
    RouteArgs ra;
    ra.T = a.T;
    ra.E = a.E;
    ra.lpad = route_lpad(a.E);
    ra.k = a.k;
    ra.renormalize = a.renormalize;
    ra.nblk = nblk;
    ra.epw = ((a.E + 16 * 4 - 1) / (16 * 4)) * 4;  // experts per wave in the scan: 16 waves, multiple of 4
    const LogitBufs lb = logit_bufs(a, noisy);
    ra.H = lb.H;
    ra.CL = lb.CL;
    ra.SG = lb.SG;
    ra.topk_idx = a.topk_idx;
    ra.topk_gate = a.topk_gate;
    ra.logits_out = a.logits_out;
    ra.part_prob = a.part_prob;
    ra.part_imp = a.part_imp;
    ra.part_load = a.part_load;
    ra.part_cnt = a.part_cnt;
    const int kk = noisy ? (a.k + 1 < a.E ? a.k + 1 : a.E) : a.k;
    err = noisy ? launch_select<true>(kk, ra, s) : launch_select<false>(kk, ra, s);
    if (err != hipSuccess) return err;
  }
  if (a.defer_tail) return hipSuccess;
  hipLaunchKernelGGL(route_reduce_kernel, dim3((a.E + kReduceThreads / 64 - 1) / (kReduceThreads / 64)),
                     dim3(kReduceThreads), 0, s, a.part_prob, a.part_imp, a.part_load, a.part_cnt,
                     nblk, a.E, a.counts_routed, a.red);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.aux_out) {
    hipLaunchKernelGGL(route_aux_kernel, dim3(1), dim3(kReduceThreads), 0, s, a.counts_routed, a.red, a.E, a.T,
                       a.k, noisy ? 1 : 0, a.aux_out);
    err = hipGetLastError();
  }
  return err;
}

// Canonical logits only (H, and for the noisy gate the clean logits and softplus
// values) into a.lg, [T][lpad] each, using a.wc for the widened weights.
hipError_t launch_route_logits(const RouteLaunch& a, hipStream_t s) {
  using namespace moe;
  if (a.T <= 0) return hipSuccess;
  const bool noisy = a.w_noise != nullptr;
  return a.dtype == 1 ? launch_logits<uint16_t>(a, noisy, s) : launch_logits<float>(a, noisy, s);
}

int route_logit_pad(int E) { return moe::route_lpad(E); }

hipError_t launch_softplus(const float* z, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe::softplus_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, out, n);
  return hipGetLastError();
}
