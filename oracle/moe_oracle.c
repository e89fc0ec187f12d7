/*
 * moe_oracle.c -- plain, slow CPU oracle for the forward pass of one
 * sparsely-gated Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or constant with the GPU library; the two are written independently
 * from the same definitions.
 *
 * Sources (the pages), cited by title and section:
 *   [Shazeer]  "Outrageously Large Neural Networks: The Sparsely-Gated
 *              Mixture-of-Experts Layer" summary page: section "Methode (mit den
 *              Schluesselgleichungen)" -- the layer equation, the "Noisy Top-K
 *              Gating" equations and the "Load-Balancing-Losses" equations.
 *   [Switch]   "Switch Transformer" dictionary page: the definition (top-1
 *              routing) and its pseudo-implementation listing (softmax over all
 *              experts, top-1, gate = mask * weights, per-expert dispatch).
 *   [Tables]   "moe paper models" page, table 2: capacity factors (1.25 ST-MoE,
 *              1/1.5/2x MegaBlocks, 2 GLaM).
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function. Routing decisions (which experts a token picks, ranks, drops) are
 * integers decided by floating-point comparisons; both this oracle and the GPU
 * take them on fp32 logits defined bit-for-bit below (canonical order of
 * operations), so the integer outputs must agree exactly. All other float
 * steps are evaluated in fp64 here.
 *
 * Parity pins: every function is pinned by tests against closed forms,
 * invariants, library routines or brute force (tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_RELU = 0, OR_GELU = 1 };

/* ------------------------------------------------------------------------ */
/* Element access: bf16 is widened to fp32 exactly (its bits are the high    */
/* half of the fp32 pattern).                                                */
/* ------------------------------------------------------------------------ */
static float widen_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float elem(const void* base, int dtype, int64_t i) {
  if (dtype == OR_BF16) return widen_bf16(((const uint16_t*)base)[i]);
  return ((const float*)base)[i];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Canonical softplus.                                                       */
/*                                                                           */
/* [Shazeer] "Noisy Top-K Gating": the noise scale is Softplus of the noise  */
/* projection, and it enters the logits that decide top-k. The pages fix no  */
/* precision, so softplus is *defined* here from correctly rounded IEEE fp32 */
/* +, -, *, /, fma, rint and ldexp only (no library transcendental), so that */
/* the CPU and the GPU evaluate the identical function:                      */
/*   softplus(z) = z                      for z > 20                         */
/*               = z + log1p(exp(-|z|))   for 0 < z <= 20                    */
/*               = log1p(exp(-|z|))       for z <= 0                         */
/* exp(y), y <= 0: Cody-Waite reduction y = n*ln2 + r with ln2 split into a  */
/* 12-bit-short head and a tail, then the degree-7 Taylor polynomial of e^r  */
/* evaluated by Horner with fma, scaled by 2^n. Zero below -87.              */
/* log1p(v), 0 <= v <= 1: log1p(v) = 2*atanh(s), s = v/(2+v), with atanh(s)  */
/* = s * sum_{j=0..8} s^(2j)/(2j+1) by Horner in s^2 with fma.               */
/* ------------------------------------------------------------------------ */
static float ln2_head(void) {
  /* ln 2 rounded to fp32, with its 12 low significand bits cleared so that
   * n*head is exact for |n| < 2^12. */
  float l = (float)0.69314718055994530942;
  uint32_t u;
  memcpy(&u, &l, sizeof u);
  u &= 0xFFFFF000u;
  memcpy(&l, &u, sizeof l);
  return l;
}

float oracle_exp_nonpos(float y) {
  if (y < -87.0f) return 0.0f;
  const float log2e = (float)1.44269504088896340736;
  const float hi = ln2_head();
  const float lo = (float)(0.69314718055994530942 - (double)hi);
  float n = rintf(y * log2e);
  float r = fmaf(-n, hi, y);
  r = fmaf(-n, lo, r);
  /* coefficients 1/i! rounded to fp32, i = 7 .. 0 */
  static const double inv_fact[8] = {1.0, 1.0, 1.0 / 2, 1.0 / 6, 1.0 / 24, 1.0 / 120, 1.0 / 720, 1.0 / 5040};
  float p = (float)inv_fact[7];
  for (int i = 6; i >= 0; --i) p = fmaf(p, r, (float)inv_fact[i]);
  return ldexpf(p, (int)n);
}

float oracle_log1p_unit(float v) {
  float s = v / (2.0f + v);
  float s2 = s * s;
  float q = (float)(1.0 / 17.0);
  for (int j = 7; j >= 0; --j) q = fmaf(q, s2, (float)(1.0 / (2 * j + 1)));
  return (s + s) * q;
}

float oracle_softplus(float z) {
  if (z > 20.0f) return z;
  float v = oracle_exp_nonpos(-fabsf(z));
  float r = oracle_log1p_unit(v);
  return z > 0.0f ? z + r : r;
}

void oracle_softplus_n(const float* z, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_softplus(z[i]);
}

void oracle_exp_nonpos_n(const float* y, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_nonpos(y[i]);
}

void oracle_log1p_unit_n(const float* v, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_log1p_unit(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Gate logits.                                                              */
/* [Shazeer] "Noisy Top-K Gating": H(x)_i = (x W_g)_i + N(0,1) *             */
/* Softplus((x W_noise)_i); the plain gate is H = x W_g ([Switch] listing:   */
/* a linear router layer). Canonical fp32 order (the reading that makes the  */
/* top-k decision reproducible): each dot product starts at +0 and adds      */
/* x[j]*W[j][e] for j = 0, 1, ..., d-1 with one fused multiply-add per term. */
/* An optional per-expert bias b[e] (used to skew routing) is added after    */
/* the sum with one rounding; the noise term is fma(eps, softplus, clean).   */
/* Outputs, all [T,E] fp32: clean logits, noise scale sigma (noisy only) and */
/* H. sigma and w_noise/noise may be NULL for the plain gate (then H=clean). */
/* ------------------------------------------------------------------------ */
/* Hot loops are built twice (baseline x86-64 and Haswell FMA/AVX2) and the
 * loader picks one by CPU; fmaf rounds once either way. */
#define ORACLE_HOT __attribute__((target_clones("default", "arch=haswell")))

ORACLE_HOT void oracle_gate_logits(int64_t T, int d, int E, int dtype, const void* x, const void* w_gate,
                        const float* gate_bias, const void* w_noise, const float* noise,
                        float* clean, float* sigma, float* H) {
  float* wg = (float*)malloc(sizeof(float) * (size_t)d * (size_t)E);
  float* wn = w_noise ? (float*)malloc(sizeof(float) * (size_t)d * (size_t)E) : NULL;
  for (int64_t i = 0; i < (int64_t)d * E; ++i) {
    wg[i] = elem(w_gate, dtype, i);
    if (wn) wn[i] = elem(w_noise, dtype, i);
  }
#pragma omp parallel
  {
    float* xr = (float*)malloc(sizeof(float) * (size_t)d);
    float* acc = (float*)malloc(sizeof(float) * (size_t)E);
    float* accn = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < d; ++j) xr[j] = elem(x, dtype, t * d + j);
      for (int e = 0; e < E; ++e) acc[e] = accn[e] = 0.0f;
      for (int j = 0; j < d; ++j) {
        const float xj = xr[j];
        const float* wrow = wg + (size_t)j * E;
        for (int e = 0; e < E; ++e) acc[e] = fmaf(xj, wrow[e], acc[e]);
        if (wn) {
          const float* nrow = wn + (size_t)j * E;
          for (int e = 0; e < E; ++e) accn[e] = fmaf(xj, nrow[e], accn[e]);
        }
      }
      for (int e = 0; e < E; ++e) {
        float c = gate_bias ? acc[e] + gate_bias[e] : acc[e];
        clean[t * E + e] = c;
        if (wn) {
          float sg = oracle_softplus(accn[e]);
          if (sigma) sigma[t * E + e] = sg;
          H[t * E + e] = fmaf(noise[t * E + e], sg, c);
        } else {
          H[t * E + e] = c;
        }
      }
    }
    free(xr);
    free(acc);
    free(accn);
  }
  free(wg);
  free(wn);
}

/* ------------------------------------------------------------------------ */
/* Top-k order.                                                              */
/* [Shazeer] KeepTopK keeps the k largest entries of H; [Switch] top-1 on    */
/* the softmax, which orders experts exactly as H does. Ties are not         */
/* treated on the pages; reading: the lower expert index wins (-0 == +0).    */
/* Writes the first kk experts of the order (H descending, index ascending). */
/* Precondition: H finite.                                                   */
/* ------------------------------------------------------------------------ */
void oracle_topk_order(int64_t T, int E, int kk, const float* H, int32_t* order) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* h = H + t * E;
    for (int s = 0; s < kk; ++s) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        int taken = 0;
        for (int q = 0; q < s; ++q)
          if (order[t * kk + q] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || h[e] > h[best]) best = e; /* strict '>' keeps the lower index on ties */
      }
      order[t * kk + s] = best;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Gate values, fp64.                                                        */
/* renormalize = 1: [Shazeer] G = Softmax(KeepTopK(H, k)) -- the softmax     */
/*   over the k kept logits, g_s = exp(H_s - H_0) / sum_s' exp(H_s' - H_0).  */
/* renormalize = 0: [Switch] listing, gate = mask * softmax(logits): the raw */
/*   full-softmax probability of each kept expert.                           */
/* prob (optional, [T,E]): the full softmax over all E experts.              */
/* ------------------------------------------------------------------------ */
void oracle_gates(int64_t T, int E, int k, int renormalize, const float* H, const int32_t* topk_idx,
                  double* gates, double* prob) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* h = H + t * E;
    double m = -INFINITY;
    for (int e = 0; e < E; ++e)
      if ((double)h[e] > m) m = h[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp((double)h[e] - m);
    if (prob)
      for (int e = 0; e < E; ++e) prob[t * E + e] = exp((double)h[e] - m) / z;
    const int32_t* idx = topk_idx + t * k;
    if (renormalize) {
      double h0 = h[idx[0]];
      double zk = 0.0;
      for (int s = 0; s < k; ++s) zk += exp((double)h[idx[s]] - h0);
      for (int s = 0; s < k; ++s) gates[t * k + s] = exp((double)h[idx[s]] - h0) / zk;
    } else {
      for (int s = 0; s < k; ++s) gates[t * k + s] = exp((double)h[idx[s]] - m) / z;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Smooth load estimator, fp64 ([Shazeer] "Load-Balancing-Losses"):          */
/*   P(x,i) = Phi((clean_i - kth_excluding(H, k, i)) / sigma_i),             */
/* where clean is the noise-free logit (x W_g, plus bias if any) and         */
/* kth_excluding(H, k, i) is the k-th largest H_j over j != i. That is the   */
/* (k+1)-th largest overall when i is in the top k, else the k-th largest.   */
/* With k == E there is no (k+1)-th value and P = 1 for every expert.        */
/* order: [T, kk] with kk = min(k+1, E). Writes load[E] = sum_x P(x, i).     */
/* ------------------------------------------------------------------------ */
static double std_normal_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

void oracle_load(int64_t T, int E, int k, const float* clean, const float* sigma, const float* H,
                 const int32_t* order, int kk, double* load) {
  for (int e = 0; e < E; ++e) load[e] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const int32_t* o = order + t * kk;
    double thr_out = H[t * E + o[k - 1]];
    int have_in = kk > k;
    double thr_in = have_in ? (double)H[t * E + o[k]] : -INFINITY;
    for (int e = 0; e < E; ++e) {
      int in_topk = 0;
      for (int s = 0; s < k; ++s)
        if (o[s] == e) in_topk = 1;
      double p;
      if (in_topk && !have_in) {
        p = 1.0;
      } else {
        double thr = in_topk ? thr_in : thr_out;
        p = std_normal_cdf(((double)clean[t * E + e] - thr) / (double)sigma[t * E + e]);
      }
      load[e] += p;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Balancing losses (unweighted; the caller applies its weights).            */
/* [Shazeer] "Load-Balancing-Losses": Importance(X) = sum over the batch of  */
/*   G(x); L = w * CV(.)^2. CV is read as population std / mean; CV^2 = 0    */
/*   for E = 1.                                                              */
/* [Switch] names an auxiliary load-balancing loss without a formula; the    */
/*   reading is the Switch Transformer paper's E * sum_e f_e * P_e with f_e  */
/*   the fraction of the T*k assignments routed to e (before capacity drops) */
/*   and P_e the batch mean of the full-softmax probability of e.            */
/* aux[0] = switch loss, aux[1] = CV^2(importance), aux[2] = CV^2(load) or   */
/* NaN when load is NULL.                                                    */
/* ------------------------------------------------------------------------ */
static double cv_squared(const double* v, int E) {
  if (E <= 1) return 0.0;
  double mean = 0.0;
  for (int e = 0; e < E; ++e) mean += v[e];
  mean /= E;
  double var = 0.0;
  for (int e = 0; e < E; ++e) var += (v[e] - mean) * (v[e] - mean);
  var /= E;
  return var / (mean * mean);
}

void oracle_aux(int64_t T, int E, int k, const int32_t* counts_routed, const double* prob_sum,
                const double* importance, const double* load, double* aux) {
  double s = 0.0;
  for (int e = 0; e < E; ++e) {
    double f = (double)counts_routed[e] / ((double)T * (double)k);
    double P = prob_sum[e] / (double)T;
    s += f * P;
  }
  aux[0] = (double)E * s;
  aux[1] = cv_squared(importance, E);
  aux[2] = load ? cv_squared(load, E) : NAN;
}

/* ------------------------------------------------------------------------ */
/* Capacity. [Tables] give capacity factors only, no formula. Reading:       */
/* C = ceil(cf * k * T / E) evaluated in double; cf <= 0 means no limit; an  */
/* explicit capacity >= 0 overrides the factor. Returns -1 for no limit.     */
/* ------------------------------------------------------------------------ */
int64_t oracle_capacity(int64_t T, int E, int k, double capacity_factor, int64_t capacity) {
  if (capacity >= 0) return capacity;
  if (!(capacity_factor > 0.0)) return -1;
  return (int64_t)ceil(capacity_factor * (double)k * (double)T / (double)E);
}

/* ------------------------------------------------------------------------ */
/* Dispatch: group the T*k assignments by expert ([Switch] listing, per      */
/* expert gather; [Shazeer] "Methode": computation is skipped where the gate */
/* is zero). Walk tokens in order and, inside a token, its slots in order;   */
/* each assignment takes the next rank of its expert; ranks >= C are        */
/* dropped (overflow dropped in token order). counts_kept = min(routed, C);  */
/* offsets = exclusive prefix sum of counts_kept over experts (E+1 entries); */
/* slot_dest[t,s] = offsets[e] + rank for kept assignments, else -1;         */
/* row_src[slot] = t. Rows of the permuted batch are therefore sorted by     */
/* (expert, token). C < 0 means no limit.                                    */
/* slot_major = 1: first-choice priority (the GShard row of [Tables]: top-2  */
/* with a capacity; reading: every token's first choice is served before any */
/* token's second choice). The walk is then slots outer, tokens inner, so    */
/* ranks -- and rows within an expert -- follow (slot, token) order.         */
/* ------------------------------------------------------------------------ */
void oracle_dispatch(int64_t T, int E, int k, int64_t C, int slot_major, const int32_t* topk_idx,
                     int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets, int32_t* slot_dest,
                     int32_t* row_src) {
  int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* rank = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T * k > 0 ? T * k : 1));
  if (slot_major) {
    for (int s = 0; s < k; ++s)
      for (int64_t t = 0; t < T; ++t) {
        int e = topk_idx[t * k + s];
        rank[t * k + s] = fill[e]++;
      }
  } else {
    for (int64_t t = 0; t < T; ++t)
      for (int s = 0; s < k; ++s) {
        int e = topk_idx[t * k + s];
        rank[t * k + s] = fill[e]++;
      }
  }
  int64_t acc = 0;
  for (int e = 0; e < E; ++e) {
    counts_routed[e] = (int32_t)fill[e];
    int64_t kept = (C >= 0 && fill[e] > C) ? C : fill[e];
    counts_kept[e] = (int32_t)kept;
    offsets[e] = (int32_t)acc;
    acc += kept;
  }
  offsets[E] = (int32_t)acc;
  for (int64_t t = 0; t < T; ++t)
    for (int s = 0; s < k; ++s) {
      int e = topk_idx[t * k + s];
      int64_t r = rank[t * k + s];
      if (C >= 0 && r >= C) {
        slot_dest[t * k + s] = -1;
      } else {
        int64_t slot = offsets[e] + r;
        slot_dest[t * k + s] = (int32_t)slot;
        row_src[slot] = (int32_t)t;
      }
    }
  free(fill);
  free(rank);
}

/* ------------------------------------------------------------------------ */
/* Expert feed-forward network, fp64 ([Shazeer] abstract and "Methode":      */
/* experts are feed-forward sub-networks). Reading: two layers without       */
/* biases, y = act(x W1[e]) W2[e], act = ReLU or the exact GELU              */
/* 0.5 z (1 + erf(z / sqrt 2)). Evaluates n rows: row r applies expert       */
/* expert[r] to row x_row[r] of x [*, d]. out: [n, d] fp64.                  */
/* ------------------------------------------------------------------------ */
ORACLE_HOT void oracle_expert_ffn_rows(int64_t n, int d, int f, int dtype, int act, const void* x, const int32_t* x_row,
                            const int32_t* expert, const void* w1, const void* w2, double* out) {
#pragma omp parallel
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
      const int64_t t = x_row[r];
      const int64_t e = expert[r];
      for (int i = 0; i < f; ++i) h[i] = 0.0;
      for (int j = 0; j < d; ++j) {
        const double xj = elem(x, dtype, t * d + j);
        const int64_t base = (e * d + j) * (int64_t)f;
        for (int i = 0; i < f; ++i) h[i] += xj * (double)elem(w1, dtype, base + i);
      }
      for (int i = 0; i < f; ++i) {
        double z = h[i];
        h[i] = (act == OR_RELU) ? (z > 0.0 ? z : 0.0) : 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
      }
      double* o = out + r * d;
      for (int j = 0; j < d; ++j) o[j] = 0.0;
      for (int i = 0; i < f; ++i) {
        const double hi = h[i];
        const int64_t base = (e * f + i) * (int64_t)d;
        for (int j = 0; j < d; ++j) o[j] += hi * (double)elem(w2, dtype, base + j);
      }
    }
    free(h);
  }
}

/* ------------------------------------------------------------------------ */
/* Combine ([Shazeer] "Methode": y = sum_i G(x)_i E_i(x); [Switch] listing:  */
/* the per-expert outputs are added back at their tokens). For each token t */
/* in tokens[], y[t] = sum over kept slots s (slot order) of                 */
/* gate[t,s] * Yp[slot_dest[t,s]]. A dropped slot contributes nothing and    */
/* surviving gates are not rescaled; a token with every slot dropped gets a  */
/* zero row. yp_row_of_slot maps a slot index to a row of yp (identity when  */
/* NULL), so a caller can pass only the rows it evaluated.                   */
/* ------------------------------------------------------------------------ */
void oracle_combine(int64_t n_tokens, const int32_t* tokens, int d, int k, const int32_t* slot_dest,
                    const double* gates, const double* yp, const int32_t* yp_row_of_slot, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_tokens; ++i) {
    const int64_t t = tokens[i];
    double* o = y + i * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    for (int s = 0; s < k; ++s) {
      const int32_t slot = slot_dest[t * k + s];
      if (slot < 0) continue;
      const int64_t row = yp_row_of_slot ? yp_row_of_slot[slot] : slot;
      const double g = gates[t * k + s];
      for (int j = 0; j < d; ++j) o[j] += g * yp[row * d + j];
    }
  }
}

/* ======================================================================== */
/* Backward pass of the layer (the pages are about training: [Shazeer]      */
/* "Fragen": the top-k is taken before the softmax, so the kept gate values */
/* keep continuous derivatives and gradients flow back through the gate;    */
/* "Kernideen": the noise term gives smooth, backpropagatable gradients).   */
/* The discrete choices (top-k sets, ranks, drops) are constants of the     */
/* backward; everything else is differentiated exactly, in fp64.            */
/* ======================================================================== */

#define ORACLE_PI 3.14159265358979323846

/* d act(z) / dz: ReLU -> 1 for z > 0 (0 at z = 0); exact GELU z Phi(z) ->   */
/* Phi(z) + z phi(z).                                                        */
static double act_grad(int act, double z) {
  if (act == OR_RELU) return z > 0.0 ? 1.0 : 0.0;
  const double phi = exp(-0.5 * z * z) / sqrt(2.0 * ORACLE_PI);
  return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * phi;
}

/* Expert FFN backward, fp64, for n rows (row r: expert expert[r] applied to */
/* x[x_row[r]]). dout[r] = dL/d(expert output of row r). Writes the expert  */
/* outputs o[r] (the forward, recomputed) and dx_rows[r] = dL/dx through    */
/* this row, and accumulates the weight gradients of every expert:          */
/*   z = x W1[e], h = act(z), o = h W2[e];                                   */
/*   dh = W2[e] dout, dz = dh * act'(z), dx = W1[e] dz,                      */
/*   dW2[e] += h^T dout, dW1[e] += x^T dz.                                   */
/* Experts run in parallel; each expert's rows are taken in row order, so   */
/* the sums do not depend on the thread count. dw1 = dw2 = NULL skips the   */
/* weight gradients.                                                         */
void oracle_expert_bwd_rows(int64_t n, int d, int f, int E, int dtype, int act, const void* x, const int32_t* x_row,
                            const int32_t* expert, const void* w1, const void* w2, const double* dout, double* o,
                            double* dx_rows, double* dw1, double* dw2) {
  const int want_dw = dw1 != NULL && dw2 != NULL; /* NULL: outputs and dx only */
  if (want_dw) {
    memset(dw1, 0, sizeof(double) * (size_t)E * d * f);
    memset(dw2, 0, sizeof(double) * (size_t)E * f * d);
  }
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* z = (double*)malloc(sizeof(double) * (size_t)f);
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    double* dz = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
      const int64_t w1b = (int64_t)e * d * f, w2b = (int64_t)e * f * d;
      for (int64_t r = 0; r < n; ++r) {
        if (expert[r] != e) continue;
        const int64_t t = x_row[r];
        for (int j = 0; j < d; ++j) xr[j] = elem(x, dtype, t * d + j);
        for (int i = 0; i < f; ++i) z[i] = 0.0;
        for (int j = 0; j < d; ++j)
          for (int i = 0; i < f; ++i) z[i] += xr[j] * (double)elem(w1, dtype, w1b + (int64_t)j * f + i);
        for (int i = 0; i < f; ++i)
          h[i] = (act == OR_RELU) ? (z[i] > 0.0 ? z[i] : 0.0) : 0.5 * z[i] * (1.0 + erf(z[i] / sqrt(2.0)));
        const double* go = dout + r * d;
        double* orow = o + r * d;
        for (int j = 0; j < d; ++j) orow[j] = 0.0;
        for (int i = 0; i < f; ++i) {
          double dh = 0.0;
          for (int j = 0; j < d; ++j) {
            const double w = (double)elem(w2, dtype, w2b + (int64_t)i * d + j);
            orow[j] += h[i] * w;
            dh += w * go[j];
            if (want_dw) dw2[w2b + (int64_t)i * d + j] += h[i] * go[j];
          }
          dz[i] = dh * act_grad(act, z[i]);
        }
        double* dxr = dx_rows + r * d;
        for (int j = 0; j < d; ++j) {
          double s = 0.0;
          for (int i = 0; i < f; ++i) {
            s += (double)elem(w1, dtype, w1b + (int64_t)j * f + i) * dz[i];
            if (want_dw) dw1[w1b + (int64_t)j * f + i] += xr[j] * dz[i];
          }
          dxr[j] = s;
        }
      }
    }
    free(xr);
    free(z);
    free(h);
    free(dz);
  }
}

/* Gate backward, fp64, per token. Inputs: the gate's H, clean and sigma     */
/* (noisy) [T,E] as the forward computed them, its noise eps [T,E], the     */
/* order [T,kk] (first kk experts, kk = min(k+1, E) when noisy, else k), the */
/* gates g [T,k] and dL/dg [T,k] (all k assignments, kept or dropped: the   */
/* caller folds in the importance loss), the routed counts and the loss     */
/* weight w_switch of E * sum_e f_e P_e, and dL/dLoad [E] (noisy). Writes   */
/* dclean [T,E] = dL/d(x W_g + b) and, noisy, du [T,E] = dL/d(x W_noise).   */
/* The T rows may be a subset of the batch of T_batch tokens (the switch   */
/* loss' f_e and P_e are batch means).                                      */
/*   renormalize: g = softmax over the kept logits -> dH_{e_s} +=            */
/*     g_s (dg_s - sum_s' g_s' dg_s');                                       */
/*   raw: g_s = p_{e_s} with p = softmax(H) over all E: dp_{e_s} += dg_s;    */
/*   switch loss: dp_j += w_switch * E * f_j / T; then dH_j += p_j (dp_j -   */
/*     sum_i p_i dp_i);                                                     */
/*   load: P(t,e) = Phi((clean_e - H_{j*}) / sigma_e), j* the expert whose  */
/*     H is kth_excluding(H, k, e) (none when e is kept and k = E):         */
/*     c = dLoad_e phi(z) / sigma_e -> dclean_e += c, dH_{j*} -= c,          */
/*     dsigma_e -= c z;                                                     */
/*   H = clean + eps sigma -> dclean += dH, dsigma += eps dH;               */
/*   sigma = softplus(u), sigmoid(u) = 1 - exp(-sigma) -> du = dsigma (1 -   */
/*     exp(-sigma)).                                                         */
void oracle_gate_bwd(int64_t T, int64_t T_batch, int E, int k, int renormalize, const float* H, const float* clean,
                     const float* sigma, const float* eps, const int32_t* order, int kk, const double* g,
                     const double* dg, const int32_t* counts_routed, double w_switch, const double* dload,
                     double* dclean, double* du) {
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    double* dp = (double*)malloc(sizeof(double) * (size_t)E);
    double* dH = (double*)malloc(sizeof(double) * (size_t)E);
    double* dcl = (double*)malloc(sizeof(double) * (size_t)E);
    double* dsig = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const float* h = H + t * E;
      const int32_t* o = order + t * kk;
      double m = -INFINITY;
      for (int e = 0; e < E; ++e)
        if ((double)h[e] > m) m = h[e];
      double zsum = 0.0;
      for (int e = 0; e < E; ++e) zsum += exp((double)h[e] - m);
      for (int e = 0; e < E; ++e) {
        p[e] = exp((double)h[e] - m) / zsum;
        dp[e] = dH[e] = dcl[e] = dsig[e] = 0.0;
      }
      const double* gt = g + t * k;
      const double* dgt = dg + t * k;
      if (renormalize) {
        double s = 0.0;
        for (int q = 0; q < k; ++q) s += gt[q] * dgt[q];
        for (int q = 0; q < k; ++q) dH[o[q]] += gt[q] * (dgt[q] - s);
      } else {
        for (int q = 0; q < k; ++q) dp[o[q]] += dgt[q];
      }
      if (w_switch != 0.0)
        for (int e = 0; e < E; ++e)
          dp[e] += w_switch * (double)E * ((double)counts_routed[e] / ((double)T_batch * (double)k)) / (double)T_batch;
      double sp = 0.0;
      for (int e = 0; e < E; ++e) sp += p[e] * dp[e];
      for (int e = 0; e < E; ++e) dH[e] += p[e] * (dp[e] - sp);
      if (sigma && dload) {
        for (int e = 0; e < E; ++e) {
          int in_topk = 0;
          for (int q = 0; q < k; ++q)
            if (o[q] == e) in_topk = 1;
          if (in_topk && kk <= k) continue; /* k == E: P = 1, no gradient */
          const int js = in_topk ? o[k] : o[k - 1];
          const double sg = sigma[t * E + e];
          const double zz = ((double)clean[t * E + e] - (double)h[js]) / sg;
          const double c = dload[e] * exp(-0.5 * zz * zz) / sqrt(2.0 * ORACLE_PI) / sg;
          dcl[e] += c;
          dH[js] -= c;
          dsig[e] -= c * zz;
        }
      }
      for (int e = 0; e < E; ++e) {
        dclean[t * E + e] = dcl[e] + dH[e];
        if (sigma) {
          const double ds = dsig[e] + (double)eps[t * E + e] * dH[e];
          du[t * E + e] = ds * (1.0 - exp(-(double)sigma[t * E + e]));
        }
      }
    }
    free(p);
    free(dp);
    free(dH);
    free(dcl);
    free(dsig);
  }
}

/* ======================================================================== */
/* Standard-normal noise of the noisy gate ([Shazeer] "Noisy Top-K Gating":  */
/* StandardNormal()), as a counter-based stream that any IEEE machine         */
/* reproduces bit for bit. Element (row, col) under key `seed`:               */
/*   words = Philox4x32-10(counter = (col, row low 32 bits, row high 32 bits, */
/*           0), key = (seed low, seed high)) -- the counter-based generator  */
/*           of Salmon, Moraes, Dror and Shaw ("Parallel Random Numbers: As   */
/*           Easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64-bit      */
/*           multiplies (0xD2511F53, 0xCD9E8D57) and xors with the key, the   */
/*           key bumped by (0x9E3779B9, 0xBB67AE85) between rounds;          */
/*   u1 = ((w0 >> 8) + 1) 2^-24 in (0, 1], u2 = (w1 >> 8) 2^-24 in [0, 1);   */
/*   z  = sqrt(-2 ln u1) cos(2 pi u2)   (Box-Muller),                         */
/* with ln and cos defined from correctly rounded fp32 +, -, *, /, fma and    */
/* sqrt only: ln u1 = log1p(u1 - 1) for u1 >= 1/2, else e ln2 + log1p(m - 1)  */
/* for u1 = m 2^e, m in [1, 2) (the canonical log1p above, whose series also  */
/* holds on [-1/2, 0]; ln2 split into the same head and tail), and            */
/* cos(2 pi u2) folded by symmetry to cos or sin of an angle in [0, pi/4]     */
/* evaluated by Taylor polynomials (degree 10 and 11) in Horner form.         */
/* ======================================================================== */
static void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
  }
}

static float ln_unit(float u) { /* u in [2^-24, 1] */
  /* u >= 1/2: ln u = log1p(u - 1), u - 1 in [-1/2, 0] exact (the series of the  */
  /* canonical log1p converges as fast there); the split below would cancel   */
  if (u >= 0.5f) return oracle_log1p_unit(u - 1.0f);
  uint32_t b;
  memcpy(&b, &u, sizeof b);
  const int e = (int)(b >> 23) - 127;
  const uint32_t mb = (b & 0x7FFFFFu) | (127u << 23);
  float m;
  memcpy(&m, &mb, sizeof m);
  const float lg = oracle_log1p_unit(m - 1.0f);
  const float hi = ln2_head();
  const float lo = (float)(0.69314718055994530942 - (double)hi);
  const float fe = (float)e;
  const float t = fmaf(fe, lo, lg);
  return fe * hi + t;
}

static float cos_two_pi(float u) { /* u in [0, 1) */
  float w = u >= 0.5f ? u - 1.0f : u; /* [-0.5, 0.5), exact */
  float a = fabsf(w);
  float sign = 1.0f;
  if (a > 0.25f) {
    a = 0.5f - a;
    sign = -1.0f;
  }
  const float two_pi = (float)6.28318530717958647692;
  float p;
  if (a > 0.125f) { /* cos(2 pi a) = sin(2 pi (1/4 - a)) */
    const float y = two_pi * (0.25f - a);
    const float y2 = y * y;
    float q = (float)(1.0 / 39916800.0);
    q = fmaf(q, -y2, (float)(1.0 / 362880.0));
    q = fmaf(q, -y2, (float)(1.0 / 5040.0));
    q = fmaf(q, -y2, (float)(1.0 / 120.0));
    q = fmaf(q, -y2, (float)(1.0 / 6.0));
    q = fmaf(q, -y2, 1.0f);
    p = y * q;
  } else {
    const float y = two_pi * a;
    const float y2 = y * y;
    float q = (float)(1.0 / 3628800.0);
    q = fmaf(q, -y2, (float)(1.0 / 40320.0));
    q = fmaf(q, -y2, (float)(1.0 / 720.0));
    q = fmaf(q, -y2, (float)(1.0 / 24.0));
    q = fmaf(q, -y2, 0.5f);
    p = fmaf(q, -y2, 1.0f);
  }
  return sign * p;
}

float oracle_normal_from_words(uint32_t w0, uint32_t w1) {
  const float u1 = (float)((w0 >> 8) + 1u) * 0x1p-24f;
  const float u2 = (float)(w1 >> 8) * 0x1p-24f;
  const float r = sqrtf(-2.0f * ln_unit(u1));
  return r * cos_two_pi(u2);
}

void oracle_philox_words(uint64_t seed, int64_t row0, int64_t rows, int cols, uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      const uint64_t row = (uint64_t)(row0 + r);
      uint32_t ctr[4] = {(uint32_t)c, (uint32_t)row, (uint32_t)(row >> 32), 0u};
      philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
      memcpy(out + 4 * (r * cols + c), ctr, sizeof ctr);
    }
}

void oracle_normal_noise(uint64_t seed, int64_t row0, int64_t rows, int cols, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      const uint64_t row = (uint64_t)(row0 + r);
      uint32_t ctr[4] = {(uint32_t)c, (uint32_t)row, (uint32_t)(row >> 32), 0u};
      philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
      out[r * cols + c] = oracle_normal_from_words(ctr[0], ctr[1]);
    }
}

void oracle_normal_from_words_n(const uint32_t* words, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_normal_from_words(words[2 * i], words[2 * i + 1]);
}

/* the two fp32 pieces of the transform, element-wise (tests) */
void oracle_ln_unit_n(const float* u, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ln_unit(u[i]);
}
void oracle_cos_two_pi_n(const float* u, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = cos_two_pi(u[i]);
}
