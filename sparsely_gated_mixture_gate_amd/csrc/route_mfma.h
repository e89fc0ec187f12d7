#pragma once

// route_mfma.h -- the gate on the bf16 MFMA units, with a certified top-k.
//
// Method (Shazeer et al. summary page, "Methode": Noisy Top-K Gating; "Switch
// Transformer" page: softmax over all experts, top-1): H = x W_g (+ b)
// (+ eps * Softplus(x W_noise)), G = Softmax(KeepTopK(H, k)) or the softmax
// probability of the kept experts.
//
// The routing decision is defined on the canonical fp32 logits (each logit an
// ascending-j fma chain from +0). Bit-for-bit, that chain needs the fp32 VALU;
// this kernel instead computes the logits with bf16 MFMAs (x and the weights
// are bf16, so every product p_j = x_j w_j is exact and only the order of the
// fp32 sums differs) and proves, token by token, that the canonical top-k is
// the same. Running-error bound (u = 2^-24, M = ceil(d / 32) MFMA k-steps,
// acc_m = the MFMA accumulator after step m, S = sum_j |p_j|, Q = sum_m |acc_m|):
//   * canonical chain s_j = fl(s_{j-1} + p_j): |s_d - sum p| <= u sum_j |s_j|, and
//     sum_j |s_j| <= (32 sum_m |exact partial after 32m terms| + 32 S) / (1 - d u);
//   * MFMA: assume each step adds its 32 products to the accumulator with an
//     error of at most 64 u (|acc_{m-1}| + sum of the step's |p_j|) (32 roundings,
//     even truncating ones, or one alignment per product), so the exact partial
//     sums are within 64 u (Q + S) of the acc_m;
//   together |acc_M - s_d| <= 96 u (Q + S)(1 + 64 u M) / (1 - d u), used as
//   B = 100 u (Q + S)(1 + 256 u M). S comes from a second MFMA on the
// sign-cleared operands in the same pass; Q is summed after every step. The
// bias add, the softplus (within 16 ulp of the true function, 1-Lipschitz) and
// the fma with eps add their own rounding terms. If, for the top-(k+1) MFMA
// values v_1 >= ..., every gap v_r - v_{r+1} (r = 1..k) exceeds twice the
// token's largest B, the canonical values keep the same order and the same
// top-k set, so the token's routing is the canonical one. Other tokens
// recompute, with the canonical chains inside the block, the logits of the
// experts that can still be in the canonical top-(k+1) (MFMA value within 2B of
// the (k+1)-th), or their whole rows (always when the caller asks for the
// fallback), and are selected again. Gate values use the MFMA logits where they
// were not recomputed (their deviation from the canonical-logit gates is a
// rounding-level effect, far inside the bf16 output tolerance).
//
// One block = 64 tokens, 512 threads (8 waves):
//   GEMM: x tile [64][BK] and weight tile [BK][NCOL] per stage in an LDS ring
//   (direct-to-LDS buffer loads): BK = 64 and up to 4 stages for NCOL <= 128
//   (each token's 128 bytes of a stage are one L2 request in lane order; each
//   load takes 8 rows 8 apart into a 1 KB block padded by 16 bytes), else
//   BK = 32 and up to 8 stages (x rows XOR-swizzled); v_mfma_f32_16x16x32_bf16 with
//   swapped operands (lane = 4 consecutive columns of one token); noisy: each
//   wave's 64 columns are 32 experts' gate columns and the same experts' noise
//   columns, so one lane holds both halves of an expert's logit.
//   Epilogue: bias, softplus, H, bound; H to LDS, per-token max bound.
//   Selection, merge, certification, fallback, per-expert partial sums as in
//   route_select (route.hip).
#include "common.h"
#include "lds_dma.h"
#include "route_common.h"

#include <type_traits>

namespace moe {

struct FusedArgs {
  int64_t T;
  int d, E, k, renormalize, nblk, force_fallback, lpad, tpb;
  const uint16_t* x;
  const uint16_t* wcat;
  const uint16_t* wt;  // noisy: wcat transposed, [NCOL][d]
  const float* bias;
  const float* noise;
  int32_t* topk_idx;
  float* topk_gate;
  float* CL;  // [T][lpad] clean logits (noisy)
  float* SG;  // [T][lpad] softplus of the noise logits (noisy)
  float* part_prob;
  float* part_imp;
  float* part_load;
  int32_t* part_cnt;
  float* dbg;  // or null: [2][T][E] the MFMA logits and their bounds (MOE_GATE_EXPORT)
};

namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTok = 64;     // rows of the logit tile (a block routes 64 tokens, or 32)


__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }  // x tile: 4 chunks per row

// Fast functions for the approximate (MFMA-logit) path: gates, probabilities
// and load estimates of certified tokens, which are compared within tolerance.
__device__ __forceinline__ float fast_exp(float y) { return __builtin_amdgcn_exp2f(y * 1.4426950408889634f); }
// softplus within 2^-20 + 2^-21 SP(z) of the true function (hardware exp2 / log2)
__device__ __forceinline__ float fast_softplus(float z) {
  if (z > 20.0f) return z;
  const float v = fast_exp(-fabsf(z));
  const float r = __builtin_amdgcn_logf(1.0f + v) * 0.69314718055994531f;
  return fmaxf(z, 0.0f) + r;
}
// Phi(z) = erfc(-z / sqrt 2) / 2 with erfc from Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7)
__device__ __forceinline__ float fast_normal_cdf(float z) {
  const float a = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
  float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  const float q = p * t * fast_exp(-(a * a));  // erfc(a)
  return z >= 0.0f ? 1.0f - 0.5f * q : 0.5f * q;
}
// Weight tile: even XOR inside the row's BCR chunks, from k mod 4 (the four rows of one
// transposing read) and bit 3 of k (rows 8 apart, read by the neighbouring 16-lane group).
// With 8 chunks (128-byte rows) bit 3 flips chunk bit 1, which moves the odd groups onto
// the 16 bank slots the even groups leave free.
template <int BCR>
__device__ __forceinline__ int swz_w(int k) {
  if constexpr (BCR == 8) return (2 * (k & 3)) ^ (((k >> 3) & 1) << 1);
  return (2 * ((k & 3) | (((k >> 3) & 1) << 2))) & (BCR - 2);
}

// wait until at most rem stages (of ld loads each) of this wave are in flight
template <int MAXREM>
__device__ __forceinline__ void wait_stages(int ld, int rem) {
  switch (ld) {
    case 1: wait_tiles<1, MAXREM>(rem); break;
    case 2: wait_tiles<2, MAXREM>(rem); break;
    case 3: wait_tiles<3, MAXREM>(rem); break;
    case 4: wait_tiles<4, MAXREM>(rem); break;
    default: wait_tiles<5, MAXREM>(rem); break;
  }
}


// Exchanges inside aligned groups of 8 lanes (DPP: quad_perm lane^1, quad_perm lane^2,
// half-row mirror lane -> 7 - lane): after the three steps every lane of the group
// holds the combination of the group's 8 values.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
  const int oi = dpp_mov<CTRL>(i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
__device__ __forceinline__ void best8(float& v, int& i) {  // first in (value desc, index asc)
  best_step<kDppXor1>(v, i);
  best_step<kDppXor2>(v, i);
  best_step<kDppHalfMirror>(v, i);
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor2>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(v))));
}
// the same over a whole wave: the four 16-lane rows by DPP (row mirror lane -> 15 - lane
// joins the two 8-lane halves), then the rows' results read from lanes 0, 16, 32, 48
constexpr int kDppRowMirror = 0x140;
__device__ __forceinline__ void best64(float& v, int& i) {
  best8(v, i);
  best_step<kDppRowMirror>(v, i);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r));
    const int oi = __builtin_amdgcn_readlane(i, r);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  v = bv;
  i = bi;
}
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(dpp_mov<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_mov<kDppXor2>(__float_as_int(v)));
  return v + __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(v)));
}
// value of lane ^ 32 / lane ^ 16 (v_permlane32_swap / v_permlane16_swap of two copies:
// the first result holds the low half / even rows twice, the second the high half /
// odd rows twice)
__device__ __forceinline__ int xor32(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? (int)r[0] : (int)r[1];
}
__device__ __forceinline__ float xor32(float v) { return __int_as_float(xor32(__float_as_int(v))); }
__device__ __forceinline__ int xor16(int v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? (int)r[0] : (int)r[1];
}
__device__ __forceinline__ float xor16(float v) { return __int_as_float(xor16(__float_as_int(v))); }
__device__ __forceinline__ float sum64(float v) {
  v = sum8(v);
  v += __int_as_float(dpp_mov<kDppRowMirror>(__float_as_int(v)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <int EP, bool NOISY, int KK>
__global__ __launch_bounds__(512) void route_fused_kernel(FusedArgs a) {
  constexpr int NCOL = NOISY ? 2 * EP : EP;
  constexpr int NI = NCOL == 64 ? 2 : 4;   // 16-column MFMA tiles per wave
  constexpr int WN_W = NCOL / (16 * NI);   // waves along columns
  constexpr int WM_W = 8 / WN_W;           // waves along tokens
  constexpr int MI = 4 / WM_W;             // 16-token MFMA tiles per wave
  constexpr int BCR = NCOL / 8;            // 16-byte chunks per weight row
  // k per LDS stage: 64 where the weight tile stays small (then the x rows of a stage are
  // 128 bytes, loaded in lane order so that each is one L2 request), else 32 (x rows swizzled)
  constexpr int SBK = NCOL <= 128 ? 64 : 32;
  constexpr int XR = SBK / 8;              // x chunks per row per stage
  constexpr int A_CH = kTok * XR;          // x chunks per stage
  constexpr int B_CH = SBK * BCR;          // weight chunks per stage
  constexpr int CH = A_CH + B_CH;
  constexpr int NR = (CH + 511) / 512;     // load rounds per stage
  // 64-wide stages: the x rows of a stage are one load round, each wave's load taking the
  // 8 rows w, w + 8, ..., w + 56 (each row's 128 bytes in lane order) into a 1 KB block of
  // its own padded to 1040 bytes, so the 16 rows of an MFMA operand read fall 16 bytes
  // apart in the banks instead of on the same ones
  constexpr int APAD = SBK == 64 ? 8 : 0;  // uint4 of padding per stage
  constexpr int STG = CH + APAD;           // uint4 per stage
  static_assert(SBK != 64 || A_CH == 512, "x rows of a 64-wide stage: one load round");
  constexpr int HS = EP + 1;               // LDS row stride of the logit tile (floats)
  constexpr int EPW = EP / 8;              // experts per wave in the scan
  constexpr int KS = KK < 8 ? KK : 8;      // selectable slots
  constexpr int RS = 24;                   // res floats per token: m, S, thr_out, thr_in, sel[8], gate[8], pad
  static_assert(CH % 64 == 0 && WN_W * WM_W == 8 && MI >= 1 && (!NOISY || NI == 4), "shape");
  // GEMM ring depth: as many stages as fit beside the other LDS use (at most 8 of 32 k, 4 of 64 k)
  constexpr int kMaxStages = SBK == 64 ? 4 : 8;
  constexpr int kStages = (144 * 1024) / (STG * 16) < kMaxStages ? (144 * 1024) / (STG * 16) : kMaxStages;
  static_assert(kStages >= 3, "ring");
  constexpr int RING = kStages * STG * 16;
  // After the GEMM the ring's LDS holds: the logit tile H and the per-token
  // results (live to the end), then the selection state, which the fallback's
  // own ring overwrites (the selection is redone after it).
  constexpr int OFF_RES = kTok * HS * 4;
  constexpr int OFF_CV = OFF_RES + kTok * RS * 4;
  constexpr int OFF_CI = OFF_CV + 8 * KK * 64 * 4;
  static_assert(OFF_CV % 16 == 0, "fallback ring must start on a 16-byte boundary");
  constexpr int OFF_WM = OFF_CI + 8 * KK * 64 * 4;
  constexpr int OFF_WS = OFF_WM + 8 * 64 * 4;
  constexpr int OFF_PART = OFF_WS + 8 * 64 * 4;
  constexpr int POST = OFF_PART + 4 * 512 * 4;
  constexpr int SMEM0 = RING > POST ? RING : POST;
  // fallback ring, from OFF_CV on: per stage the weight tile [F_BK][NCOL] and
  // the x rows of 16 flagged tokens [16][F_BK]; F_BK = 64, 32, 16 or 8 rows, the
  // largest of which 3 stages fit (fewer stages, fewer barriers along the chains).
  // A block that holds more than half the LDS runs alone on its CU anyway, so its
  // fallback ring may grow to 152 KB.
  constexpr int FR = 16;  // tokens per fallback round
  constexpr int F_FREE = (SMEM0 > 80 * 1024 ? 152 * 1024 : SMEM0) - OFF_CV;
  constexpr int F_BK = F_FREE / ((64 * BCR + FR * 8) * 16) >= 3   ? 64
                       : F_FREE / ((32 * BCR + FR * 4) * 16) >= 3 ? 32
                       : F_FREE / ((16 * BCR + FR * 2) * 16) >= 3 ? 16
                                                                  : 8;
  constexpr int F_CPR = F_BK / 8;                // x chunks per row per stage
  constexpr int F_WCH = F_BK * BCR;              // weight chunks per stage
  constexpr int F_XCH = FR * F_CPR;              // x chunks per stage
  constexpr int F_CH = F_WCH + F_XCH;            // chunks per fallback stage
  constexpr int F_NR = (F_CH + 511) / 512;
  constexpr int F_STAGES = F_FREE / (F_CH * 16) < 8 ? F_FREE / (F_CH * 16) : 8;
  constexpr int SMEM_R = SMEM0 > OFF_CV + F_STAGES * F_CH * 16 ? SMEM0 : OFF_CV + F_STAGES * F_CH * 16;
  // The candidate chains stage their operands from OFF_CV + 4 KB on, in whatever LDS
  // the occupancy leaves: up to 152 KB for a block alone on its CU, else 77 KB (two
  // blocks per CU).
  constexpr int SMEM_F = SMEM0 > 80 * 1024 ? 152 * 1024 : 77 * 1024;
  constexpr int SMEM = SMEM_R > SMEM_F ? SMEM_R : SMEM_F;
  static_assert(F_WCH % 64 == 0 && F_STAGES >= 3 && F_NR <= 5 && NR <= 5 &&
                    SMEM + 1024 <= 160 * 1024,
                "LDS");
  __shared__ uint4 smem_u4[SMEM / 16];
  __shared__ float bmax_s[kTok];
  __shared__ int flist_s[kTok];
  __shared__ int flag_s[kTok];  // token row not certified
  __shared__ int nflag_s;
  __shared__ int fb_full_s;  // the candidate pairs do not fit: the block recomputes whole rows
  __shared__ int np_s;       // candidate pairs of the block
  __shared__ int tslot_s[kTok];  // token row of each x-row slot of a staging round
  __shared__ int rnd_s[2];       // end of the staging round's pairs, its token count
  char* smem = reinterpret_cast<char*>(smem_u4);
  float* Hs = reinterpret_cast<float*>(smem);
  float* cand_v = reinterpret_cast<float*>(smem + OFF_CV);
  int* cand_i = reinterpret_cast<int*>(smem + OFF_CI);
  float* wmax = reinterpret_cast<float*>(smem + OFF_WM);
  float* wsum = reinterpret_cast<float*>(smem + OFF_WS);
  float* res = reinterpret_cast<float*>(smem + OFF_RES);
  float* part = reinterpret_cast<float*>(smem + OFF_PART);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d, E = a.E, k = a.k;
  const int64_t T = a.T;
  // tokens t0 .. t0 + rows - 1 (a.tpb = 64, or 32 when 64-token blocks would leave
  // CUs idle; the tile is 64 rows either way, rows past `rows` are clamped copies)
  const int64_t t0 = (int64_t)blockIdx.x * a.tpb;
  const int rows = (int)min<int64_t>(a.tpb, T - t0);
  if (tid < kTok) bmax_s[tid] = 0.0f;
  if (tid == 0) fb_full_s = 0;

  // ---- GEMM: V = x W and S = |x| |W| over the block's 64 tokens ----------------
  const int32x4 rsX = buffer_rsrc(a.x + t0 * d, (uint32_t)rows * d * 2);
  const int32x4 rsW = buffer_rsrc(a.wcat, (uint32_t)d * NCOL * 2);
  int voff[NR];
  bool isA[NR], act[NR];
  int ld = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int c = tid + 512 * i;
    act[i] = (i * 512 + wave * 64) < CH;  // wave-uniform
    isA[i] = (i * 512 + wave * 64) < A_CH;
    ld += act[i] ? 1 : 0;
    if (c < A_CH) {
      const int row = SBK == 64 ? wave + 8 * (lane >> 3) : c / XR;
      const int p = SBK == 64 ? lane & 7 : c % XR;
      const int pc = SBK == 64 ? p : p ^ swz4(row);
      voff[i] = min(row, rows - 1) * d * 2 + (pc << 4);  // rows past T: clamped, never stored
    } else {
      const int b = c - A_CH;
      const int kr = b / BCR, p = b % BCR;
      voff[i] = kr * NCOL * 2 + ((p ^ swz_w<BCR>(kr)) << 4);  // rows past d load zero
    }
  }
  const uint32_t lds0 = lds_address(&smem_u4[0]);
  // The stage offset goes into the per-lane offset so the whole offset is
  // range-checked: x chunks past d in the last stage meet zero weight rows.
  auto issue = [&](int kt) {
    const int st = kt % kStages;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (!act[i]) continue;
      const uint32_t dst = lds0 + (uint32_t)(st * STG * 16 + (SBK == 64 && isA[i] ? wave * 1040 : (i * 512 + wave * 64 + APAD) * 16));
      if (isA[i])  // token rows: read by this block alone, once (non-temporal)
        load_to_lds_nt(__builtin_amdgcn_readfirstlane(dst), voff[i] + kt * SBK * 2, rsX, 0);
      else
        load_to_lds(__builtin_amdgcn_readfirstlane(dst), voff[i] + kt * SBK * NCOL * 2, rsW, 0);
    }
  };

  const int wm = wave / WN_W, wn = wave % WN_W;
  // 16-token MFMA row tiles of this wave that hold tokens of the block (the tile has
  // 64 rows; 32-token blocks and the last block leave the rest idle)
  const int mact = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * 16 * MI + 15) / 16)));
  const int g = lane >> 4, s = lane & 15;
  // acc: the logits; qs: Q + S, i.e. |acc| after every k-step (the step before
  // this one; the last is added after the loop) plus the sign-cleared MFMA
  floatx4 acc[MI][NI], qs[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = qs[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // PART: only the first mact row tiles hold tokens (a compile-time switch, so full
  // tiles keep a branch-free loop)
  auto add_q = [&](auto part_c) {
    constexpr bool PART = decltype(part_c)::value;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (PART && i >= mact) break;
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) qs[i][j][r] += fabsf(acc[i][j][r]);
    }
  };

  auto compute = [&](int st, auto part_c) {
    constexpr bool PART = decltype(part_c)::value;
    const uint4* sA = &smem_u4[st * STG];
    lds_char* sB = (lds_char*)(&smem_u4[st * STG + A_CH + APAD]);
#pragma unroll
    for (int ks = 0; ks < SBK / 32; ++ks) {  // one 32-wide MFMA k-step each
      add_q(part_c);
      uint4 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (PART && mi >= mact) break;
        const int row = wm * (16 * MI) + mi * 16 + s;
        af[mi] = SBK == 64 ? sA[(row & 7) * 65 + (row >> 3) * 8 + ks * 4 + g] : sA[row * XR + (g ^ swz4(row))];
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        // transposing read: lane L of a 16-lane group receives W[k0 .. k0+3][n + L]
        const int krow = ks * 32 + 8 * g + (s >> 2);
        const int ncol = wn * (16 * NI) + ni * 16 + 4 * (s & 3);
        const int c = ncol >> 3;
        const int b0 = krow * (NCOL * 2) + ((c ^ swz_w<BCR>(krow)) << 4) + ((ncol & 7) << 1);
        const int b1 = (krow + 4) * (NCOL * 2) + ((c ^ swz_w<BCR>(krow + 4)) << 4) + ((ncol & 7) << 1);
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sB + b0));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sB + b1));
        const short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bfr[ni] = __builtin_bit_cast(uint4, both);
      }
      const uint4 m7 = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (PART && mi >= mact) break;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[ni]),
                                                                __builtin_bit_cast(bf16x8, af[mi]), acc[mi][ni], 0, 0, 0);
          qs[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[ni] & m7),
                                                               __builtin_bit_cast(bf16x8, af[mi] & m7), qs[mi][ni], 0, 0, 0);
        }
      }
    }
  };

  const int nk = (d + SBK - 1) / SBK;  // stages
  const int nsteps = nk * (SBK / 32);  // 32-wide MFMA k-steps, M of the bound
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < nk) issue(t);
  auto main_loop = [&](auto part_c) {
    for (int kt = 0; kt < nk; ++kt) {
      wait_stages<kStages - 2>(ld, min(kStages - 2, nk - 1 - kt));
      block_barrier();
      if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
      compute(kt % kStages, part_c);
    }
    add_q(part_c);
  };
  if (mact == MI) main_loop(std::false_type{});
  else main_loop(std::true_type{});
  __syncthreads();  // the ring is dead from here on; its LDS holds the logit tile and the selection state

  // ---- epilogue: clean logit (+ bias), softplus, H and the bound ------------------
  // Bound of |acc_mfma - acc_canon|: KB * (Q + S) (see the file header).
  const float KB = 100.0f * 0x1.0p-24f * (1.0f + 256.0f * 0x1.0p-24f * (float)nsteps) * 1.004f;
  // noise of this lane's (token, expert) entries, all loads in flight together
  constexpr int NE = NOISY ? NI / 2 : NI;  // 16-expert groups per lane
  float epsv[MI][NE][4];
  if constexpr (NOISY) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi >= mact) break;
      const int64_t t = t0 + min(wm * (16 * MI) + mi * 16 + s, rows - 1);
#pragma unroll
      for (int ni = 0; ni < NE; ++ni) {
        const int e = 32 * wn + 16 * ni + 4 * g;
        if ((E & 3) == 0 && e < E) {
          const float4 v = *reinterpret_cast<const float4*>(a.noise + t * E + e);
          epsv[mi][ni][0] = v.x; epsv[mi][ni][1] = v.y; epsv[mi][ni][2] = v.z; epsv[mi][ni][3] = v.w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) epsv[mi][ni][j] = e + j < E ? a.noise[t * E + e + j] : 0.0f;
        }
      }
    }
  }
  // the gate bias of this lane's experts (the same for all its token rows), loaded once
  float biasv[NE][4];
#pragma unroll
  for (int ni = 0; ni < NE; ++ni) {
    const int e0 = NOISY ? 32 * wn + 16 * ni + 4 * g : wn * (16 * NI) + ni * 16 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) biasv[ni][j] = (a.bias && e0 + j < E) ? a.bias[e0 + j] : 0.0f;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = wm * (16 * MI) + mi * 16 + s;  // token row of this lane
    const int64_t t = t0 + m;
    if (mi >= mact) {  // no token in this row tile: its logit rows are never selected
#pragma unroll
      for (int ni = 0; ni < NE; ++ni) {
        const int e0 = NOISY ? 32 * wn + 16 * ni + 4 * g : wn * (16 * NI) + ni * 16 + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e0 + j < EP) Hs[m * HS + e0 + j] = -INFINITY;
      }
      continue;
    }
    float bmax = 0.0f;
#pragma unroll
    for (int ni = 0; ni < NE; ++ni) {
      const int e0 = NOISY ? 32 * wn + 16 * ni + 4 * g : wn * (16 * NI) + ni * 16 + 4 * g;
      float clv[4], spv[4], hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + j;
        float cl = acc[mi][ni][j];
        if (a.bias && e < E) cl = cl + biasv[ni][j];
        const float bcl = KB * qs[mi][ni][j] * (1.0f + 0x1.0p-22f) + 0x1.0p-22f * fabsf(cl);
        float h = cl, bh = bcl, sp = 0.0f;
        if constexpr (NOISY) {
          const float zn = acc[mi][ni + 2][j];
          sp = fast_softplus(zn);
          const float eps = epsv[mi][ni][j];
          h = __builtin_fmaf(eps, sp, cl);
          // |fast_softplus(a) - canon_softplus(b)| <= |a - b| + 2^-19 SP + 2^-20 (both within their error of SP)
          const float bn = KB * qs[mi][ni + 2][j];
          const float bsp = bn * (1.0f + 0x1.0p-18f) + 0x1.0p-18f * sp + 0x1.0p-20f;
          bh = (fabsf(eps) * bsp + bcl) * (1.0f + 0x1.0p-22f) + 0x1.0p-22f * fabsf(h);
        }
        clv[j] = cl;
        spv[j] = sp;
        hv[j] = e < E ? h : -INFINITY;
        if (e < E) bmax = fmaxf(bmax, bh);
        if (a.dbg && e < E && m < rows) {  // the certificate's inputs, for auditing
          a.dbg[t * E + e] = h;
          a.dbg[(a.T + t) * E + e] = bh;
        }
        if (e < EP) Hs[m * HS + e] = hv[j];
      }
      if constexpr (NOISY) {
        if (m < rows && e0 < E) {
          if (e0 + 3 < E) {
            *reinterpret_cast<float4*>(a.CL + t * a.lpad + e0) = float4{clv[0], clv[1], clv[2], clv[3]};
            *reinterpret_cast<float4*>(a.SG + t * a.lpad + e0) = float4{spv[0], spv[1], spv[2], spv[3]};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (e0 + j < E) {
                a.CL[t * a.lpad + e0 + j] = clv[j];
                a.SG[t * a.lpad + e0 + j] = spv[j];
              }
          }
        }
      }
    }
    // lanes s, s+16, s+32, s+48 share the token row: max over them, then over waves
    bmax = fmaxf(bmax, xor16(bmax));
    bmax = fmaxf(bmax, xor32(bmax));
    if (g == 0) atomicMax(reinterpret_cast<int*>(&bmax_s[m]), __float_as_int(bmax));  // non-negative floats order as ints
  }
  __syncthreads();

  // ---- selection over the logit tile in LDS ---------------------------------------
  // phase 1, lane = token: this wave's experts [wave*EPW, +EPW): top-KK, max, sum of exp
  auto scan = [&]() {
    const int e_lo = min(E, wave * EPW), e_hi = min(E, e_lo + EPW);
    const float* hrow = Hs + lane * HS;
    float bv[KK];
    int bi[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7FFFFFFF;
    }
    float hv[EPW];  // all of this wave's logits of the token, read before the comparisons
#pragma unroll
    for (int c = 0; c < EPW; ++c) hv[c] = e_lo + c < e_hi ? hrow[e_lo + c] : -INFINITY;
#pragma unroll
    for (int c = 0; c < EPW; ++c) {
      if (e_lo + c >= e_hi) break;
      float v = hv[c];
      int i = e_lo + c;
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
    const float m_w = bv[0];
    float s_w = 0.0f;
#pragma unroll
    for (int c = 0; c < EPW; ++c)
      if (e_lo + c < e_hi) s_w += fast_exp(hv[c] - m_w);
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      cand_v[(wave * KK + r) * 64 + lane] = bv[r];
      cand_i[(wave * KK + r) * 64 + lane] = bi[r];
    }
    wmax[wave * 64 + lane] = e_lo < e_hi ? m_w : -INFINITY;
    wsum[wave * 64 + lane] = s_w;
  };

  // phase 1 for blocks of at most 32 tokens: lane = (token lane % 32, half lane / 32)
  // of this wave's experts, so all 64 lanes scan; each lane then inserts the other
  // half's sorted top-KK (the top-KK under value desc, index asc is the same in any
  // insertion order) and the two partial softmax sums are rescaled to the wave max.
  auto scan_halves = [&]() {
    constexpr int EH = EPW / 2;
    const int tl = lane & 31, h = lane >> 5;
    const int w_lo = min(E, wave * EPW), w_hi = min(E, w_lo + EPW);
    const int e_lo = min(w_hi, w_lo + h * EH), e_hi = min(w_hi, e_lo + EH);
    const float* hrow = Hs + tl * HS;
    float bv[KK];
    int bi[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7FFFFFFF;
    }
    auto insert = [&](float v, int i) {
      if (!better(v, i, bv[KK - 1], bi[KK - 1])) return;
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
    };
    float hv[EH];
#pragma unroll
    for (int c = 0; c < EH; ++c) hv[c] = e_lo + c < e_hi ? hrow[e_lo + c] : -INFINITY;
#pragma unroll
    for (int c = 0; c < EH; ++c)
      if (e_lo + c < e_hi) insert(hv[c], e_lo + c);
    const float m_h = bv[0];
    float s_h = 0.0f;
#pragma unroll
    for (int c = 0; c < EH; ++c)
      if (e_lo + c < e_hi) s_h += fast_exp(hv[c] - m_h);
    const bool have_h = e_lo < e_hi;
    const bool have_o = xor32((int)have_h) != 0;
    const float m_o = xor32(m_h), s_o = xor32(s_h);
    float ov[KK];
    int oi[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      ov[r] = xor32(bv[r]);
      oi[r] = xor32(bi[r]);
    }
#pragma unroll
    for (int r = 0; r < KK; ++r)
      if (oi[r] != 0x7FFFFFFF) insert(ov[r], oi[r]);
    const float m_w = bv[0];
    const float s_w = (have_h ? s_h * fast_exp(m_h - m_w) : 0.0f) + (have_o ? s_o * fast_exp(m_o - m_w) : 0.0f);
    // every lane writes its token's lists (lanes 32..63 into slots no token uses)
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      cand_v[(wave * KK + r) * 64 + lane] = bv[r];
      cand_i[(wave * KK + r) * 64 + lane] = bi[r];
    }
    wmax[wave * 64 + lane] = w_lo < w_hi ? m_w : -INFINITY;
    wsum[wave * 64 + lane] = s_w;
  };

  // token row tl's results from its top-KK values / indices (value desc, index asc),
  // softmax max m and sum S: gates, load-estimator thresholds, outputs
  auto finish = [&](int tl, const float (&sel_v)[KK], const int (&sel_i)[KK], float m, float S) {
    const int64_t t = t0 + tl;
    float gt[8];
    if (a.renormalize) {
      float den = 0.0f, num[8];
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        if (q >= k) break;
        num[q] = fast_exp(sel_v[q] - sel_v[0]);
        den += num[q];
      }
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        if (q >= k) break;
        gt[q] = num[q] / den;
      }
    } else {
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        if (q >= k) break;
        gt[q] = fast_exp(sel_v[q] - m) / S;
      }
    }
    float thr_out = 0.0f, thr_in = 0.0f;
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      if (r == k - 1) thr_out = sel_v[r];
      if (r == k) thr_in = sel_v[r];
    }
    float* rt = res + tl * RS;
    rt[0] = m;
    rt[1] = 1.0f / S;
    rt[2] = thr_out;
    rt[3] = thr_in;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      if (q >= k) break;
      reinterpret_cast<int*>(rt)[4 + q] = sel_i[q];
      rt[12 + q] = gt[q];
      if (tl < rows) {
        a.topk_idx[t * k + q] = sel_i[q];
        a.topk_gate[t * k + q] = gt[q];
      }
    }
  };

  // phase 2, all waves: 8 lanes per token row (wave w: rows 8w .. 8w+7, lane = 8 * row
  // + list), lane j holding the sorted top-KK list of scan wave j. Each of the KK rounds
  // takes the best list head of the group (value desc, index asc; expert ids are unique
  // across the lists) and advances the list it came from; the softmax max and sum
  // combine the same way. The group's first lane certifies the row (gaps against
  // twice its largest bound) and writes its results, or flags it.
  auto merge8 = [&]() {
    const int j = lane & 7;
    const int m = wave * 8 + (lane >> 3);
    float lv[KK];
    int li[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      lv[r] = cand_v[(j * KK + r) * 64 + m];
      li[r] = cand_i[(j * KK + r) * 64 + m];
    }
    float sel_v[KK];
    int sel_i[KK];
    int h = 0;  // this list's next entry
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      float v = -INFINITY;
      int i = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < KK; ++q)
        if (q == h) {
          v = lv[q];
          i = li[q];
        }
      float bv = v;
      int bi = i;
      best8(bv, bi);
      sel_v[r] = bv;
      sel_i[r] = bi;
      if (bi != 0x7FFFFFFF && i == bi) ++h;
    }
    const float mw = wmax[j * 64 + m];
    const float mt = max8(mw);
    const float S = sum8(mw != -INFINITY ? wsum[j * 64 + m] * fast_exp(mw - mt) : 0.0f);
    if (j != 0) return;
    if (m >= rows) {  // rows past the block's tokens: nothing to route
      flag_s[m] = 0;
      return;
    }
    bool ok = !a.force_fallback;
    const float b2 = 2.0f * bmax_s[m];
    const int ngap = min(k, KK - 1);
#pragma unroll
    for (int r = 0; r + 1 < KK; ++r)
      if (r < ngap) ok = ok && (sel_v[r] - sel_v[r + 1] > b2);  // false for NaN
    flag_s[m] = ok ? 0 : 1;
    if (!ok) {
      // candidates of the canonical top-KK: every expert with v >= v_KK - 2B (see the fallback)
      res[m * RS + 20] = sel_v[KK - 1] - b2;
      return;
    }
    finish(m, sel_v, sel_i, mt, S);
  };

  // one wave, lane = expert (e = lane + 64 c): top-KK and softmax of token tl
  // from its canonical logits in H (repeated wave arg-max, value desc, index asc)
  auto reselect = [&](int tl) {
    constexpr int G = EP / 64;
    const float* hrow = Hs + tl * HS;
    float hv[G];
#pragma unroll
    for (int c = 0; c < G; ++c) hv[c] = lane + 64 * c < E ? hrow[lane + 64 * c] : -INFINITY;
    uint32_t taken = 0;
    float sel_v[KK];
    int sel_i[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      float v = -INFINITY;
      int i = 0x7FFFFFFF;
#pragma unroll
      for (int c = 0; c < G; ++c)
        if (lane + 64 * c < E && !((taken >> c) & 1u) && better(hv[c], lane + 64 * c, v, i)) {
          v = hv[c];
          i = lane + 64 * c;
        }
      best64(v, i);
      sel_v[r] = v;
      sel_i[r] = i;
      if (i != 0x7FFFFFFF && (i & 63) == lane) taken |= 1u << (i >> 6);
    }
    const float m = sel_v[0];
    float S = 0.0f;
#pragma unroll
    for (int c = 0; c < G; ++c)
      if (lane + 64 * c < E) S += fast_exp(hv[c] - m);
    S = sum64(S);
    if (lane == 0) finish(tl, sel_v, sel_i, m, S);
  };


  if (a.tpb <= 32) scan_halves();
  else scan();
  __syncthreads();
  merge8();
  __syncthreads();
  if (wave == 0) {  // flagged rows in token order
    const bool bad_l = flag_s[lane] != 0;
    const uint64_t bad = __ballot(bad_l);
    if (bad_l) flist_s[__builtin_amdgcn_mbcnt_hi((uint32_t)(bad >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bad, 0u))] = lane;
    if (lane == 0) nflag_s = __popcll(bad);
  }
  __syncthreads();

  // ---- fallback: canonical fp32 chains for the uncertified tokens ------------------
  // Rounds of 16 flagged tokens. Thread (slot f0, column c) of TPR x NCOL runs
  // the chains of tokens f0*NFG .. +NFG for column c; weight tiles and the
  // tokens' x chunks stream through a 2-stage LDS ring (direct-to-LDS loads).
  const int nflag = nflag_s;
  if (nflag > 0) {
    // A flagged token's canonical logit c_e lies within B (its largest bound) of the
    // MFMA value v_e. With V the KK-th largest v, the KK experts with v >= V have
    // c >= V - B, so an expert with v_e < V - 2B has c_e < V - B and cannot be in
    // the canonical top-KK. Only the other experts (the candidates) need their
    // canonical chains; the rest keep their MFMA logits, which then enter only the
    // softmax sums. The (token, candidate) pairs are listed in token order; in rounds
    // of as many as the LDS holds, each round's token rows and the pairs' weight
    // columns are gathered into LDS as fp32 by all threads (a token's row once, however
    // many of its pairs the round holds), and each chain is run by one thread from LDS
    // (one fma per step). The forced fallback, and blocks with more pairs than threads
    // (or than about 16 rounds), recompute whole rows instead (below).
    int* pair_tok = reinterpret_cast<int*>(smem + OFF_CV);  // [512] token row of each pair
    int* pair_e = pair_tok + 512;                            // [512] its expert (| x-row slot << 16)
    constexpr int OFF_ST = OFF_CV + 4096;                    // staged operands
    static_assert(OFF_WM - OFF_CV >= 4096 && SMEM >= OFF_ST, "candidate lists");
    constexpr int NW = NOISY ? 2 : 1;                        // weight columns per pair: gate (, noise)
    // x-row slots (d fp32) and pair blocks (NW * d weights), each padded to 16 bytes mod
    // 256 so that the chains' 16-byte reads (one pair per lane) fall on distinct banks.
    // WB16 (noisy gate): the weights stay bf16 and are widened to fp32 (exactly) in the
    // chains, one shift or mask per k, so a round holds about twice the pairs; that extra
    // op lengthens a chain by about 1.45x, which pays where rounds are short (the noise
    // column starts nofb bytes into the pair block, 128 mod 256, so the two lanes that run
    // a pair's gate and noise chains read distinct banks). Plain gates stage fp32 weights.
    constexpr bool WB16 = NOISY;
    const int nofb = NOISY ? ((2 * d + 255) / 256) * 256 + 128 : 0;
    const int xb = 4 * d + ((16 - (4 * d) % 256) + 256) % 256;
    const int wb = WB16 ? (nofb + 2 * d) + ((16 - (nofb + 2 * d) % 256) + 256) % 256 : xb;
    const int cap = SMEM - OFF_ST;
    const int maxp = (cap - xb) / wb;  // pairs of a single token that one round holds
    int* resi = reinterpret_cast<int*>(res);
    // candidates of flagged token q (lane = expert), in expert order; with emit, their
    // pairs are written from the token's list offset on; returns the count
    auto candidates = [&](int q, bool emit) -> int {
      const int m = flist_s[q];
      const float lo = res[m * RS + 20];
      const float* hrow = Hs + m * HS;
      int cnt = emit ? resi[m * RS + 22] : 0;
      const int c0 = cnt;
#pragma unroll
      for (int c = 0; c < EP / 64; ++c) {
        const int e = lane + 64 * c;
        const bool cand = e < E && !(hrow[e] < lo);  // a NaN logit or bound makes a candidate
        const uint64_t bal = __ballot(cand);
        if (emit && cand) {
          const int pos =
              cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          pair_tok[pos] = m;
          pair_e[pos] = e;
        }
        cnt += __popcll(bal);
      }
      return cnt - c0;
    };
    bool full = a.force_fallback != 0 || maxp < 1;
    if (!full) {
      for (int q = wave; q < nflag; q += 8) {
        const int cnt = candidates(q, false);
        if (lane == 0) resi[flist_s[q] * RS + 21] = cnt;
      }
      __syncthreads();
      if (wave == 0) {  // list offsets in token order
        const int c = lane < nflag ? resi[flist_s[lane] * RS + 21] : 0;
        int v = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int n = __shfl_up(v, off);
          if (lane >= off) v += n;
        }
        if (lane < nflag) resi[flist_s[lane] * RS + 22] = v - c;
        if (lane == 63) {
          np_s = v;
          fb_full_s = (v > 512 || v > 16 * maxp) ? 1 : 0;
        }
      }
      __syncthreads();
      full = fb_full_s != 0;
    }
    if (!full) {
      const int np = np_s;
      for (int q = wave; q < nflag; q += 8) candidates(q, true);
      __syncthreads();
      const int n8 = d / 8;
      for (int p0 = 0; p0 < np;) {
        // the round: pairs p0 .. p1 - 1, as many as fit with their nt token rows
        if (tid == 0) {
          int p = p0, nt = 0, last = -1;
          while (p < np) {
            const int m = pair_tok[p];
            const int nt2 = nt + (m != last ? 1 : 0);
            if (p > p0 && (nt2 * xb + (p + 1 - p0) * wb > cap || p - p0 >= 512 / NW)) break;  // NW threads per pair
            if (m != last) tslot_s[nt] = m;
            pair_e[p] = (pair_e[p] & 0xFFFF) | ((nt2 - 1) << 16);
            nt = nt2;
            last = m;
            ++p;
          }
          rnd_s[0] = p;
          rnd_s[1] = nt;
        }
        __syncthreads();
        const int p1 = rnd_s[0], nt = rnd_s[1], pr = p1 - p0;
        const int pbase = OFF_ST + nt * xb;
        // gather: item (x-row slot, 8 consecutive k) -> one 16-byte x load; item (pair,
        // 8 consecutive k) -> 8 weight loads (noisy: two 16-byte loads from the transposed
        // copy, gate and noise column); x widened to fp32, weights as bf16 (WB16) or fp32,
        // k ascending
        auto gather = [&](int it) {
          if (it < nt * n8) {
            const int sl = it / n8, j8 = it - sl * n8;
            float* blk = reinterpret_cast<float*>(smem + OFF_ST + sl * xb) + 8 * j8;
            const uint4 xv = *reinterpret_cast<const uint4*>(a.x + (t0 + tslot_s[sl]) * d + 8 * j8);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int h = 0; h < 2; ++h)
              *reinterpret_cast<float4*>(blk + 4 * h) = float4{bf16_lo(xw[2 * h]), bf16_hi(xw[2 * h]),
                                                               bf16_lo(xw[2 * h + 1]), bf16_hi(xw[2 * h + 1])};
          } else {
            const int i2 = it - nt * n8;
            const int pl = i2 / n8, j8 = i2 - pl * n8;
            const int e = pair_e[p0 + pl] & 0xFFFF;
            char* blk = smem + pbase + pl * wb + (WB16 ? 16 : 32) * j8;
            if constexpr (NOISY) {  // contiguous rows of the transposed copy: 16 bytes each of the two columns
              const size_t cg = 64 * (e >> 5) + (e & 31);
              *reinterpret_cast<uint4*>(blk) = *reinterpret_cast<const uint4*>(a.wt + cg * d + 8 * j8);
              *reinterpret_cast<uint4*>(blk + nofb) = *reinterpret_cast<const uint4*>(a.wt + (cg + 32) * d + 8 * j8);
            } else {
              const uint16_t* __restrict__ w = a.wcat + (size_t)(8 * j8) * NCOL + e;
              uint32_t wg[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) wg[u] = w[(size_t)u * NCOL];
              static_assert(!WB16, "plain gates stage fp32 weights");
              float* fb = reinterpret_cast<float*>(blk);
#pragma unroll
              for (int h = 0; h < 2; ++h)
                *reinterpret_cast<float4*>(fb + 4 * h) = float4{bf16_to_f32(wg[4 * h]), bf16_to_f32(wg[4 * h + 1]),
                                                                bf16_to_f32(wg[4 * h + 2]), bf16_to_f32(wg[4 * h + 3])};
            }
          }
        };
        const int nit = (nt + pr) * n8;
        for (int it = tid; it < nit; it += 1024) {  // two items per pass, their loads in flight together
          gather(it);
          if (it + 512 < nit) gather(it + 512);
        }
        __syncthreads();
        // one chain per thread (noisy: threads 2p and 2p + 1 run pair p's gate and noise
        // chains side by side, then the gate thread takes the noise sum from its neighbour)
        if (tid < NW * pr) {
          const int pl = NOISY ? tid >> 1 : tid;
          const int m = pair_tok[p0 + pl], pe = pair_e[p0 + pl];
          const int e = pe & 0xFFFF;
          const int64_t t = t0 + m;
          const float4* bx = reinterpret_cast<const float4*>(smem + OFF_ST + (pe >> 16) * xb);
          const char* bwc = smem + pbase + pl * wb + (NOISY ? (tid & 1) * nofb : 0);
          float acc = 0.0f;
#pragma unroll 4
          for (int j8 = 0; j8 < d / 8; ++j8) {  // k = 8 j8 .. 8 j8 + 7 in order: low half, then high half of each word
            const float4 x0 = bx[2 * j8], x1 = bx[2 * j8 + 1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float ws[8];
            if constexpr (WB16) {
              const uint4 wv = reinterpret_cast<const uint4*>(bwc)[j8];
              const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                ws[2 * u] = __uint_as_float(ww[u] << 16);
                ws[2 * u + 1] = __uint_as_float(ww[u] & 0xFFFF0000u);
              }
            } else {
              const float4 w0 = reinterpret_cast<const float4*>(bwc)[2 * j8], w1 = reinterpret_cast<const float4*>(bwc)[2 * j8 + 1];
              ws[0] = w0.x; ws[1] = w0.y; ws[2] = w0.z; ws[3] = w0.w;
              ws[4] = w1.x; ws[5] = w1.y; ws[6] = w1.z; ws[7] = w1.w;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = __builtin_fmaf(xs[u], ws[u], acc);
          }
          if constexpr (NOISY) {
            const float accn = __shfl_xor(acc, 1);  // the noise chain of the pair
            if ((tid & 1) == 0) {
              float cl = acc;
              if (a.bias) cl = cl + a.bias[e];
              const float sp = canon_softplus(accn);
              Hs[m * HS + e] = __builtin_fmaf(a.noise[t * E + e], sp, cl);
              a.CL[t * a.lpad + e] = cl;
              a.SG[t * a.lpad + e] = sp;
            }
          } else {
            float cl = acc;
            if (a.bias) cl = cl + a.bias[e];
            Hs[m * HS + e] = cl;
          }
        }
        __syncthreads();  // the staging area is refilled by the next round
        p0 = p1;
      }
    } else {
      constexpr int TPR = 512 / NCOL;  // token slots
      constexpr int NFG = FR / TPR;    // tokens per thread
      const int f0 = tid / NCOL, c = tid % NCOL;
      const int32x4 rsXall = buffer_rsrc(a.x, (uint32_t)(T * d * 2));
      const uint32_t fl0 = lds_address(&smem_u4[OFF_CV / 16]);
      uint32_t fvoff[F_NR];  // byte offsets (x offsets can pass 2^31; T*d*2 < 2^32 is checked on the host)
      bool fisW[F_NR], fact[F_NR];
      int fld = 0;
#pragma unroll
      for (int i = 0; i < F_NR; ++i) {
        fact[i] = (i * 512 + wave * 64) < F_CH;  // wave-uniform (the x chunks may fill part of a wave)
        fisW[i] = (i * 512 + wave * 64) < F_WCH;
        fld += fact[i] ? 1 : 0;
        const int cc = tid + 512 * i;
        const int kr = cc / BCR, p = cc % BCR;
        fvoff[i] = (uint32_t)(kr * NCOL * 2 + ((p ^ swz_w<BCR>(kr)) << 4));  // weight chunks (x chunks set per round)
      }
      // One round: NF tokens per thread (TPR * NF tokens), chains interleaved over
      // the tokens so consecutive fmas are independent.
      auto round = [&](int base, auto nf_tag) {
        constexpr int NF = decltype(nf_tag)::value;
        constexpr int RT = TPR * NF;  // tokens in this round
        // x chunk slots: row r of the round (token flist[base + r], or a valid row), chunk p
#pragma unroll
        for (int i = 0; i < F_NR; ++i) {
          const int cc = tid + 512 * i - F_WCH;
          if (cc >= 0) {
            const int r = min(cc / F_CPR, FR - 1), p = cc % F_CPR;  // lanes past the x chunks: any valid offset
            const int m = flist_s[min(base + r, nflag - 1)];
            fvoff[i] = (uint32_t)((t0 + m) * d * 2) + (uint32_t)(p << 4);
          }
        }
        auto fissue = [&](int kt) {
          const int st = kt % F_STAGES;
#pragma unroll
          for (int i = 0; i < F_NR; ++i) {
            if (!fact[i]) continue;
            const uint32_t dst = fl0 + (uint32_t)((st * F_CH + i * 512 + wave * 64) * 16);
            if (fisW[i]) {
              load_to_lds(__builtin_amdgcn_readfirstlane(dst), (int)(fvoff[i] + (uint32_t)(kt * F_BK * NCOL * 2)), rsW, 0);
            } else if (tid + 512 * i < F_CH) {  // x chunks: every slot loads (slots past this round's rows repeat a
                                                 // valid row), so every wave with fact[i] issues the load its waits count
              load_to_lds(__builtin_amdgcn_readfirstlane(dst), (int)(fvoff[i] + (uint32_t)(kt * F_BK * 2)), rsXall, 0);
            }
          }
        };
        float accv[NF];
#pragma unroll
        for (int q = 0; q < NF; ++q) accv[q] = 0.0f;
        const bool busy = base + f0 * NF < nflag;  // wave-uniform (a wave's columns share one token slot)
        const int fnk = (d + F_BK - 1) / F_BK;
#pragma unroll
        for (int t = 0; t < F_STAGES - 1; ++t)
          if (t < fnk) fissue(t);
        for (int kt = 0; kt < fnk; ++kt) {
          wait_stages<F_STAGES - 2>(fld, min(F_STAGES - 2, fnk - 1 - kt));
          block_barrier();  // stage kt in LDS for every wave; the buffer of stage kt-1 is free
          if (kt + F_STAGES - 1 < fnk) fissue(kt + F_STAGES - 1);
          const char* sb = smem + OFF_CV + (kt % F_STAGES) * F_CH * 16;
          lds_char* sw = (lds_char*)(&smem_u4[OFF_CV / 16 + (kt % F_STAGES) * F_CH]);
          const uint4* sx = reinterpret_cast<const uint4*>(sb + F_WCH * 16);
          const int nj = min(F_BK, d - kt * F_BK);  // a multiple of 8
          auto do_q8 = [&](int q8) {
            // column c's weights of rows 8 q8 .. +7 by two transposing reads: the lanes
            // of a 16-lane group hold 16 consecutive columns, source lane s points at
            // row 8 q8 + s/4, columns 4 (s%4) .. +3 of the group
            const int kr = q8 * 8 + ((lane & 15) >> 2);
            const int nc = (c - lane) + 16 * (lane >> 4) + 4 * (lane & 3);
            const int b0 = kr * (NCOL * 2) + (((nc >> 3) ^ swz_w<BCR>(kr)) << 4) + ((nc & 7) << 1);
            const int b1 = (kr + 4) * (NCOL * 2) + (((nc >> 3) ^ swz_w<BCR>(kr + 4)) << 4) + ((nc & 7) << 1);
            const shortx4 wlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sw + b0));
            const shortx4 whi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sw + b1));
            float wv[8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              wv[u] = bf16_to_f32((uint16_t)wlo[u]);
              wv[u + 4] = bf16_to_f32((uint16_t)whi[u]);
            }
            uint4 xv[NF];
#pragma unroll
            for (int q = 0; q < NF; ++q) xv[q] = sx[(f0 * NF + q) * F_CPR + q8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
              for (int q = 0; q < NF; ++q) {
                const uint32_t w2 = (&xv[q].x)[u >> 1];
                const float xs = (u & 1) ? bf16_hi(w2) : bf16_lo(w2);
                accv[q] = __builtin_fmaf(xs, wv[u], accv[q]);
              }
          };
          if (!busy) {
            // token slot past the flagged tokens: loads and barriers only
          } else if (nj == F_BK) {
#pragma unroll
            for (int q8 = 0; q8 < F_CPR; ++q8) do_q8(q8);  // full stage: every LDS read can be issued early
          } else {
            for (int q8 = 0; q8 < nj / 8; ++q8) do_q8(q8);
          }
        }
        block_barrier();  // the ring is reused by the next round
#pragma unroll
        for (int q = 0; q < NF; ++q) {
          const int fi = base + f0 * NF + q;
          const bool on = fi < nflag;
          const int m = flist_s[min(fi, nflag - 1)];
          const int64_t t = t0 + m;
          if constexpr (NOISY) {
            const float accn = __shfl_xor(accv[q], 32);  // column c + 32 holds the same expert's noise logit
            const int e = 32 * (c >> 6) + (c & 31);
            if (on && !(c & 32) && e < E) {
              float cl = accv[q];
              if (a.bias) cl = cl + a.bias[e];
              const float sp = canon_softplus(accn);
              const float h = __builtin_fmaf(a.noise[t * E + e], sp, cl);
              Hs[m * HS + e] = h;
              a.CL[t * a.lpad + e] = cl;
              a.SG[t * a.lpad + e] = sp;
            }
          } else {
            const int e = c;
            if (on && e < E) {
              float cl = accv[q];
              if (a.bias) cl = cl + a.bias[e];
              Hs[m * HS + e] = cl;
            }
          }
        }
        return RT;
      };
      for (int base = 0; base < nflag;) {
        const int need = (nflag - base + TPR - 1) / TPR;  // tokens per thread still needed
        if (need <= 1) base += round(base, std::integral_constant<int, 1>{});
        else if (need <= 2 || NFG < 4) base += round(base, std::integral_constant<int, (NFG < 2 ? NFG : 2)>{});
        else if (need <= 4 || NFG < 8) base += round(base, std::integral_constant<int, (NFG < 4 ? NFG : 4)>{});
        else if (need <= 8 || NFG < 16) base += round(base, std::integral_constant<int, (NFG < 8 ? NFG : 8)>{});
        else base += round(base, std::integral_constant<int, NFG>{});
      }
    }
    __syncthreads();
    for (int q = wave; q < nflag; q += 8) reselect(flist_s[q]);
    __syncthreads();
  }

  // ---- phase 3, lane = expert: sums over token slices in token order ---------------
  constexpr int G = EP / 64;   // expert groups of 64
  constexpr int TS = 8 / G;    // token slices
  const int gq = wave % G, ts = wave / G;
  const int e = gq * 64 + lane;
  if (e < E) {
    const bool have_in = KK > k;
    const int tls = (rows + TS - 1) / TS;  // tokens per slice
    const int tl_lo = min(rows, ts * tls), tl_hi = min(rows, tl_lo + tls);
    float p_sum = 0.0f, imp_sum = 0.0f, ld_sum = 0.0f;
    int cnt = 0;
    constexpr int TB = 8;  // tokens whose global loads are in flight together
    for (int tb = tl_lo; tb < tl_hi; tb += TB) {
      float cb[TB], sb[TB];
      if constexpr (NOISY) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const int64_t t = t0 + min(tb + u, tl_hi - 1);
          cb[u] = a.CL[t * a.lpad + e];
          sb[u] = a.SG[t * a.lpad + e];
        }
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int tl = tb + u;
        if (tl >= tl_hi) break;
        const float* rt = res + tl * RS;
        const float h = Hs[tl * HS + e];
        p_sum += fast_exp(h - rt[0]) * rt[1];
        bool in_k = false;
        float gk = 0.0f;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          if (q >= k) break;
          if (reinterpret_cast<const int*>(rt)[4 + q] == e) {
            in_k = true;
            gk = rt[12 + q];
          }
        }
        imp_sum += gk;
        cnt += in_k ? 1 : 0;
        if constexpr (NOISY) {
          const float thr = in_k ? rt[3] : rt[2];
          ld_sum += (in_k && !have_in) ? 1.0f : fast_normal_cdf((cb[u] - thr) * __builtin_amdgcn_rcpf(sb[u]));
        }
      }
    }
    const int o = ts * EP + e;
    part[0 * 512 + o] = p_sum;
    part[1 * 512 + o] = imp_sum;
    part[2 * 512 + o] = ld_sum;
    reinterpret_cast<int*>(part)[3 * 512 + o] = cnt;
  }
  __syncthreads();
  if (tid < E) {
    float p_sum = 0.0f, imp_sum = 0.0f, ld_sum = 0.0f;
    int cnt = 0;
    for (int q = 0; q < TS; ++q) {
      const int o = q * EP + tid;
      p_sum += part[0 * 512 + o];
      imp_sum += part[1 * 512 + o];
      ld_sum += part[2 * 512 + o];
      cnt += reinterpret_cast<const int*>(part)[3 * 512 + o];
    }
    const int64_t o = (int64_t)tid * a.nblk + blockIdx.x;
    a.part_prob[o] = p_sum;
    a.part_imp[o] = imp_sum;
    a.part_load[o] = ld_sum;
    a.part_cnt[o] = cnt;
  }
}

template <int EP, bool NOISY, int KK>
hipError_t launch_fused_t(const FusedArgs& fa, hipStream_t s) {
  hipLaunchKernelGGL((route_fused_kernel<EP, NOISY, KK>), dim3((unsigned)fa.nblk), dim3(512), 0, s, fa);
  return hipGetLastError();
}

}  // namespace

// Launch of the certified gate for EP padded experts, with or without the noise
// columns; kk = min(k + 1, E). Each (EP, NOISY) pair is instantiated in a
// translation unit of its own (route_mfma_e*.hip), so the nine top-(k+1)
// variants of each pair compile in parallel.
template <int EP, bool NOISY>
hipError_t launch_fused_kk(int kk, const FusedArgs& fa, hipStream_t s) {
  switch (kk) {
    case 1: return launch_fused_t<EP, NOISY, 1>(fa, s);
    case 2: return launch_fused_t<EP, NOISY, 2>(fa, s);
    case 3: return launch_fused_t<EP, NOISY, 3>(fa, s);
    case 4: return launch_fused_t<EP, NOISY, 4>(fa, s);
    case 5: return launch_fused_t<EP, NOISY, 5>(fa, s);
    case 6: return launch_fused_t<EP, NOISY, 6>(fa, s);
    case 7: return launch_fused_t<EP, NOISY, 7>(fa, s);
    case 8: return launch_fused_t<EP, NOISY, 8>(fa, s);
    default: return launch_fused_t<EP, NOISY, 9>(fa, s);
  }
}

}  // namespace moe
