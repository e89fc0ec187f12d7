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
