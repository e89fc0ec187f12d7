// common.h -- device helpers and launch declarations shared by the gfx950
// kernels of the MoE layer forward. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// bf16 values travel as raw 16-bit patterns (uint16_t); widening is exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest, ties to even:
// one v_cvt_pk_bf16_f32 on gfx950 (the default round mode is nearest-even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Activation of the first expert layer: ReLU, or the exact GELU 0.5 z (1 + erf(z / sqrt 2)).
template <int ACT>
__device__ __forceinline__ float activation(float z) {
  if constexpr (ACT == 0) {
    return z > 0.0f ? z : 0.0f;
  } else {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
  }
}

// GELU for bf16 outputs: erf from Abramowitz & Stegun 7.1.26 (absolute error
// <= 1.5e-7, far below bf16 rounding), branch-free, with one reciprocal and one
// exp2. With a = |z|/sqrt 2, t = 1/(1 + p a) and q = P(t) t exp(-a^2),
// erf(a) = 1 - q; then GELU(z) = z Phi(z) = max(z, 0) - h with h = |z| q / 2 for
// either sign of z (z - h for z >= 0, -h = z q / 2 for z < 0), so there is no
// cancellation for negative z. The 1/2 is folded into the coefficients of P. |z|
// is clamped at 10 inside h (h < 1e-20 there), which keeps infinite z finite.
// Both clamps are single v_med3_f32 (fminf / fmaxf would add canonicalising ops);
// the upper bound FLT_MAX of max(z, 0) turns +inf into FLT_MAX, which the bf16
// rounding of the output takes back to +inf.
__device__ __forceinline__ float gelu_fast(float z) {
  const float za = __builtin_amdgcn_fmed3f(fabsf(z), 0.0f, 10.0f);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f * 0.70710678118654752f, za, 1.0f));
  float r = __builtin_fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  r = __builtin_fmaf(r, t, 0.5f * 1.421413741f);
  r = __builtin_fmaf(r, t, 0.5f * -0.284496736f);
  r = __builtin_fmaf(r, t, 0.5f * 0.254829592f);
  r = r * t;
  const float e = __builtin_amdgcn_exp2f(za * (za * (-0.5f * 1.4426950408889634f)));
  return __builtin_fmaf(-(za * r), e, __builtin_amdgcn_fmed3f(z, 0.0f, 3.40282347e38f));
}

template <int ACT>
__device__ __forceinline__ float activation_bf16(float z) {
  if constexpr (ACT == 0) {
    return __builtin_amdgcn_fmed3f(z, 0.0f, 3.40282347e38f);  // max(z, 0) in one op (+inf: as in gelu_fast)
  } else {
    return gelu_fast(z);
  }
}

// d act(z) / dz for the backward pass: ReLU -> 1 for z > 0, else 0; exact GELU
// z Phi(z) -> Phi(z) + z phi(z), with Phi from the same erf approximation as
// gelu_fast (|error| <= 1.5e-7) and phi(z) = exp(-z^2 / 2) / sqrt(2 pi).
template <int ACT>
__device__ __forceinline__ float activation_grad(float z) {
  if constexpr (ACT == 0) {
    return z > 0.0f ? 1.0f : 0.0f;
  } else {
    const float za = __builtin_amdgcn_fmed3f(fabsf(z), 0.0f, 10.0f);
    const float a = za * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
    float r = __builtin_fmaf(1.061405429f, t, -1.453152027f);
    r = __builtin_fmaf(r, t, 1.421413741f);
    r = __builtin_fmaf(r, t, -0.284496736f);
    r = __builtin_fmaf(r, t, 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(za * (za * (-0.5f * 1.4426950408889634f)));  // exp(-z^2 / 2)
    const float q = r * t * e;                                                          // erfc(|z| / sqrt 2)
    const float cdf = z >= 0.0f ? 1.0f - 0.5f * q : 0.5f * q;
    return __builtin_fmaf(z * 0.3989422804014327f, e, cdf);
  }
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Launchers (host). Each returns the hipError_t of its launches.
// ---------------------------------------------------------------------------
struct RouteLaunch {
  int64_t T;
  int d, E, k, dtype, renormalize;
  const void* x;
  const void* w_gate;
  const float* gate_bias;
  const void* w_noise;
  const float* noise;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts_routed;
  float* aux_out;
  float* logits_out;
  // workspace pieces
  float* wc;         // [d][ncol] fp32 gate (and noise) weights in column blocks
  float* lg;         // route_logit_floats(T, E, noisy): logits H [, clean logits, softplus of noise logits]
  uint16_t* wcat;    // route_wcat_elems(d, E, noisy): bf16 gate (+ noise) weights of the MFMA gate
  int gate_mode;     // MOE_GATE_*
  bool defer_tail;   // leave the partial sums and the losses to the dispatch (forward path)
  float* part_prob;  // [E][nblk]
  float* part_imp;   // [E][nblk]
  float* part_load;  // [E][nblk]
  int32_t* part_cnt; // [E][nblk]
  double* red;       // [3][E]
};
// blocks of per-block partial sums the route writes (the gate kernels' grid)
int route_partial_blocks(int64_t T, int E, int dtype, int gate_mode, bool logits_out);
int route_fused_tokens(int64_t T);
size_t route_weight_floats(int d, int E, bool noisy);
size_t route_logit_floats(int64_t T, int E, bool noisy);
hipError_t launch_route(const RouteLaunch& a, hipStream_t s);
bool route_fused_supported(int dtype, int E);
size_t route_wcat_elems(int d, int E, bool noisy);
hipError_t launch_route_fused(const RouteLaunch& a, bool noisy, int force_fallback, float* CL, float* SG, int lpad,
                              hipStream_t s);

struct DispatchLaunch {
  int64_t T;
  int d, E, k, dtype;
  int slot_major;  // drop order: 0 token order, 1 first-choice priority (walk slot-major)
  int64_t C;  // < 0: unlimited
  int64_t max_rows;
  const void* x;
  const int32_t* topk_idx;
  int32_t* counts_kept;
  int32_t* offsets;
  int32_t* slot_dest;
  int32_t* row_src;
  void* x_perm;
  int32_t* blk_cnt;  // [E][nb] workspace
  int32_t* tile_start;  // [E+1] M-tile prefix for the expert FFN, or null
  int tile_rows;        // M-tile rows of that prefix
  bool skip_permute;    // x_perm is not written (the expert FFN gathers its rows from x)
  void* y_zero;         // top-1 layers only: y [T, d], whose rows of dropped tokens are zeroed (or null)
  // forward path (optional, route_tail): the end of the routing step -- fixed-order
  // sums of the gate's per-block partials (extra blocks of the count kernel) and
  // the losses (end of the scan kernel)
  bool route_tail;
  const float *part_prob, *part_imp, *part_load;
  const int32_t* part_cnt;
  int route_nblk;
  int32_t* counts_routed;
  double* red;
  float* aux_out;  // or null
  int noisy;
};
int64_t dispatch_num_blocks(int64_t assignments);
hipError_t launch_dispatch(const DispatchLaunch& a, hipStream_t s);

struct FfnLaunch {
  int d, f, E, dtype, act;
  int64_t max_rows;
  int64_t capacity;  // rows per expert at most (< 0: unlimited)
  const void* x_perm;
  const int32_t* offsets;
  const void* w1;
  const void* w2;
  void* y_perm;
  void* h1;             // [max_rows, f] dtype workspace
  int32_t* tile_start;  // [E+1] workspace
  bool tile_map_ready;  // tile_start already holds the M-tile prefix (built by the dispatch scan)
  // bf16 forward path (optional): layer 1 gathers row r from x_src[row_src[r]] instead of
  // x_perm[r]; with y_out set (top-1 layers), layer 2 writes gate[t] * row into
  // y_out[t], t = row_src[r], instead of y_perm[r]
  const void* x_src;
  const int32_t* row_src;
  int64_t T;
  void* y_out;
  const float* gate;
  void* mid_event;  // hipEvent_t recorded between the two layers' launches (phase timing), or null
};
hipError_t launch_expert_ffn(const FfnLaunch& a, hipStream_t s);
int ffn_tile_rows(int dtype, int64_t capacity, int64_t max_rows, int E);  // M-tile rows the FFN launch uses

struct CombineLaunch {
  int64_t T;
  int d, k, dtype;
  const void* y_perm;
  const int32_t* slot_dest;
  const float* topk_gate;
  void* y;
};
hipError_t launch_combine(const CombineLaunch& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
// The grouped products of the expert backward (bwd_gemm.hip).
enum BwdGemmKind {
  kBwdRecompute1,  // H1 = act(Xp W1[e]), D1 = act'(Xp W1[e])
  kBwdRecompute2,  // O = H1 W2[e]
  kBwdDataGrad2,   // dZ = (dO W2[e]^T) * D1
  kBwdDataGrad1,   // dXp = dZ W1[e]^T
  kBwdWeightGrad   // dW[e] = A[seg e]^T B[seg e]
};
struct BwdGemmArgs {
  const uint16_t* A;  // element pointers (fp32 layers: float data behind the same pointers)
  const uint16_t* B;
  uint16_t* C;
  uint16_t* C2;          // second output (kBwdRecompute1: act'(z))
  const uint16_t* Dmul;  // elementwise factor of the output (kBwdDataGrad2)
  const int32_t* offsets;
  const int32_t* tile_start;  // M-tile map (segments on M)
  int E, M, N, K, n_tiles_m, n_tiles_n;
  int64_t lda, ldb, ldc;                      // row strides in elements
  int64_t b_expert_stride, c_expert_stride;   // per-expert offsets of the weights / weight gradients
  uint32_t a_bytes, b_bytes;                  // extents of the A buffer and (segments on K) the B buffer
};
int bwd_gemm_tile_rows(int dtype);
int bwd_gemm_tile_cols(int dtype);
hipError_t launch_bwd_gemm(BwdGemmKind kind, const BwdGemmArgs& g, int64_t blocks, int dtype, int act, hipStream_t s);
// M-tile map of bm-row tiles over the expert segments (offsets [E+1] -> tile_start)
hipError_t launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* tile_start, hipStream_t s);

struct BwdMiscArgs {
  int64_t T;
  int d, E, k, dtype, renormalize, noisy, lpad;
  const void* x;
  const void* w_gate;
  const void* w_noise;
  const float* noise;
  const void* dy;
  const void* o;   // [R, d] recomputed expert outputs
  void* dO;        // [R, d] gate-scaled upstream rows
  const int32_t* slot_dest;
  const int32_t* topk_idx;
  const float* topk_gate;
  float* dg;       // [T, k] dL/dg from the combine
  const double* red;  // the route's fp64 per-expert sums [3][E]
  const int32_t* counts_routed;
  double w_switch, w_imp, w_load;
  float *dimp, *dload, *dpsw;  // [E] each
  const float *H, *CL, *SG;    // canonical logits, clean logits, softplus [T][lpad]
  float *dclean, *du;          // [T, E]
  const void* dxp;             // [R, d]
  void* dx;                    // [T, d]
};
hipError_t launch_bwd_gather(const BwdMiscArgs& b, hipStream_t s);
hipError_t launch_bwd_gate(const BwdMiscArgs& b, hipStream_t s);
int64_t bwd_gate_wgrad_chunks(int64_t T);
hipError_t launch_bwd_gate_wgrad(const BwdMiscArgs& b, const float* G, float* dW, float* db, float* part,
                                 float* part_b, hipStream_t s);
hipError_t launch_bwd_dx(const BwdMiscArgs& b, hipStream_t s);

// ---------------------------------------------------------------------------
// Hierarchical gate (route_hier.hip)
// ---------------------------------------------------------------------------
struct HierLaunch {
  int64_t T;
  int groups, per_group, k_group, k_expert, noisy_p, lpad_p, lpad_s;
  const float *Hp, *CLp, *SGp;  // primary logits, clean logits, softplus [T][lpad_p]
  const float* Hs;              // secondary logits [T][lpad_s], column g * per_group + j
  int32_t* order_p;             // [T][k_group + 1] primary order (workspace)
  float* gate_p;                // [T][k_group] primary gates (workspace)
  int32_t* topk_idx;            // [T][k_group * k_expert]
  float* topk_gate;
  int32_t* counts_routed;       // [groups * per_group]
  double* red;                  // [E + 2 groups]: combined importance, primary importance, primary load
  float* aux_out;               // [3] or null
};
hipError_t launch_route_hier(const HierLaunch& h, hipStream_t s);
hipError_t launch_route_logits(const RouteLaunch& a, hipStream_t s);
int route_logit_pad(int E);
