// bwd_gemm.hip -- the grouped matrix products of the layer's backward pass.
//
// Method: the backward of each expert's feed-forward network (Shazeer et al.
// summary page, abstract and "Methode": experts are feed-forward networks;
// "Fragen": gradients reach the experts and the gate through the kept gate
// values). With z = x W1[e], h = act(z), o = h W2[e] for each row of expert e's
// segment and do = dL/do:
//   recompute   h = act(Xp W1[e]) and act'(z)       (segments on M, B = W1[e] [K][N])
//   recompute   o = H1 W2[e]                        (segments on M, B = W2[e] [K][N])
//   data grad   dz = (dO W2[e]^T) * act'(z)         (segments on M, B = W2[e] read as [N][K])
//   data grad   dXp = dZ W1[e]^T                    (segments on M, B = W1[e] read as [N][K])
//   weight grad dW2[e] = H1^T dO, dW1[e] = Xp^T dZ  (segments on K: the rows of expert e)
// One kernel template covers all six: each operand is either K-contiguous in
// memory ([rows][K], read from LDS with ds_read_b128) or K-strided ([K][cols],
// read with the gfx950 transposing ds_read_b64_tr_b16), and the expert
// segment either tiles M (one M-tile list per expert, from the device-built
// tile map) or is the K range (weight gradients: one tile grid per expert).
//
// Design (gfx950): 128 x 128 x 32 tiles, 256 threads = 2 x 2 waves of 64 x 64,
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation and swapped operands (each
// lane ends with 4 consecutive output columns of one row: 8-byte stores). Both
// operand tiles go HBM -> LDS by direct-to-LDS buffer loads in their memory
// layout (16-byte chunks, XOR-swizzled), into a 4-stage ring (3 k-tiles in
// flight). Everything past the segment, K or N loads as zero without touching
// memory. fp32 layers use a plain LDS-tiled fp32 FMA kernel over the same
// index maps.
#include "common.h"
#include "lds_dma.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBM = 128, kBN = 128, kBK = 32, kStages = 4, kThreads = 256;
constexpr int kOut = 0x7FFFFFF0;  // a byte offset past any operand: the buffer load returns zero

// K-contiguous tile [128 rows][32 k]: 4 chunks per row, chunk ^ swz_kc(row).
__device__ __forceinline__ int swz_kc(int row) { return (row >> 2) & 3; }
// K-strided tile [32 k][128 cols]: 16 chunks per row, chunk ^ 2 * swz_ks(k) (the
// 8 rows of one transposing read land in 8 distinct 32-byte bank groups).
__device__ __forceinline__ int swz_ks(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// Locate M-tile mt (128 rows) of the expert-sorted rows. false past the last tile.
__device__ __forceinline__ bool find_mtile(const int32_t* __restrict__ tile_start, const int32_t* __restrict__ offsets,
                                           int E, int mt, int* e_out, int* row0, int* row_end) {
  if (mt >= tile_start[E]) return false;
  const int e = tile_start[E + 1 + mt];  // the expert of every M-tile
  *e_out = e;
  *row0 = offsets[e] + (mt - tile_start[e]) * kBM;
  *row_end = offsets[e + 1];
  return true;
}

// C = A . B per expert. A_KC / B_KC: operand is K-contiguous ([rows][K]); otherwise
// K-strided ([K][cols]). SEGK: the expert segment is the K range (weight
// gradients, one M x N grid per expert); else it tiles M (rows of the permuted
// batch). EPI: 0 store; 1 multiply by Dmul[row][col] (act'(z)) then store;
// 2 store act(acc) to C and act'(acc) to C2.
template <bool A_KC, bool B_KC, bool SEGK, int EPI, int ACT>
__global__ __launch_bounds__(kThreads) void bwd_gemm_bf16_kernel(BwdGemmArgs g) {
  constexpr int A_CH = kBM * kBK / 8, B_CH = kBN * kBK / 8;  // 16-byte chunks per tile
  constexpr int STAGE_CH = A_CH + B_CH;
  constexpr int LD = (A_CH + B_CH) / kThreads;  // loads per thread per k-tile (4)
  __shared__ uint4 smem[kStages * STAGE_CH];

  int e, row0, row_end, m0, n0, k_lo, k_hi;
  if constexpr (SEGK) {
    const int tiles = g.n_tiles_m * g.n_tiles_n;
    e = blockIdx.x / tiles;
    const int t = blockIdx.x - e * tiles;
    m0 = (t / g.n_tiles_n) * kBM;
    n0 = (t % g.n_tiles_n) * kBN;
    row0 = 0;
    row_end = g.M;
    k_lo = g.offsets[e];
    k_hi = g.offsets[e + 1];
  } else {
    const int mt = blockIdx.x / g.n_tiles_n;
    if (!find_mtile(g.tile_start, g.offsets, g.E, mt, &e, &row0, &row_end)) return;
    n0 = (blockIdx.x - mt * g.n_tiles_n) * kBN;
    m0 = row0;
    k_lo = 0;
    k_hi = g.K;
  }
  const int klen = k_hi - k_lo;
  const int nk = (klen + kBK - 1) / kBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mlim = SEGK ? g.M : row_end;  // rows (M) past this load zero and are not stored

  // operand base pointers (per expert for the weights)
  const uint16_t* Ab = g.A;
  const uint16_t* Bb = g.B + (SEGK ? 0 : (int64_t)e * g.b_expert_stride);
  const int32x4 rsA = buffer_rsrc(Ab, g.a_bytes);
  const int32x4 rsB = buffer_rsrc(Bb, SEGK ? g.b_bytes : (uint32_t)(g.b_expert_stride * 2));
  const uint32_t lds0 = lds_address(&smem[0]);

  // one operand tile: chunk c of this thread; returns the byte offset or kOut
  //   KC: tile [128 rows][32 k]: row = c / 4, k chunk = (c % 4) ^ swz_kc(row)
  //   KS: tile [32 k][128 cols]: k row = c / 16, col chunk = (c % 16) ^ 2 swz_ks(kr)
  // rows of the KC tile / cols of the KS tile are M indices for A and N indices for B.
  auto offset_of = [&](bool kc, bool is_a, int c, int kt) -> int {
    const int64_t ld = is_a ? g.lda : g.ldb;
    const int lim = is_a ? mlim : g.N;  // M (A) or N (B) extent
    const int base = is_a ? m0 : n0;
    const int kbase = k_lo + kt * kBK;
    if (kc) {
      const int row = c >> 2, kc8 = ((c & 3) ^ swz_kc(row)) * 8;
      const int gi = base + row, gk = kbase + kc8;
      if (gi >= lim || gk >= k_hi) return kOut;
      return (int)(((uint32_t)gi * (uint32_t)ld + (uint32_t)gk) * 2u);
    }
    const int kr = c >> 4, col = (((c & 15) ^ (2 * swz_ks(kr))) * 8);
    const int gk = kbase + kr, gi = base + col;
    if (gi >= lim || gk >= k_hi) return kOut;
    return (int)(((uint32_t)gk * (uint32_t)ld + (uint32_t)gi) * 2u);
  };
  auto issue = [&](int kt) {
    const int st = kt % kStages;
#pragma unroll
    for (int i = 0; i < A_CH / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const uint32_t dst = lds0 + (uint32_t)((st * STAGE_CH + i * kThreads + wave * 64) * 16);
      load_to_lds(__builtin_amdgcn_readfirstlane(dst), offset_of(A_KC, true, c, kt), rsA, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const uint32_t dst = lds0 + (uint32_t)((st * STAGE_CH + A_CH + i * kThreads + wave * 64) * 16);
      load_to_lds(__builtin_amdgcn_readfirstlane(dst), offset_of(B_KC, false, c, kt), rsB, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 64 x 64
  const int gq = lane >> 4, s = lane & 15;
  // operand fragment: 16 rows (or cols) x 8 k of MFMA tile idx of this wave
  auto frag = [&](bool kc, int stage_off, int idx16) -> bf16x8 {
    if (kc) {
      const uint4* t = &smem[stage_off];
      const int row = idx16 * 16 + s;
      return __builtin_bit_cast(bf16x8, t[row * 4 + (gq ^ swz_kc(row))]);
    }
    lds_char* t = (lds_char*)(&smem[stage_off]);
    const int krow = 8 * gq + (s >> 2);
    const int col = idx16 * 16 + 4 * (s & 3);
    const int c = col >> 3;
    const int b0 = krow * 256 + ((c ^ (2 * swz_ks(krow))) << 4) + ((col & 7) << 1);
    const int b1 = (krow + 4) * 256 + ((c ^ (2 * swz_ks(krow + 4))) << 4) + ((col & 7) << 1);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(t + b0));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(t + b1));
    const short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < nk) issue(t);
  for (int kt = 0; kt < nk; ++kt) {
    wait_tiles<LD, kStages - 2>(min(kStages - 2, nk - 1 - kt));
    block_barrier();  // tile kt is in LDS for every wave; the stage of tile kt - 1 is free
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
    const int st = kt % kStages;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(A_KC, st * STAGE_CH, wm * 4 + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag(B_KC, st * STAGE_CH + A_CH, wn * 4 + j);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  }

  // epilogue: lane holds C[m0 + wm*64 + i*16 + s][n0 + wn*64 + j*16 + 4 gq + (0..3)]
  uint16_t* C = g.C + (SEGK ? (int64_t)e * g.c_expert_stride : 0);
  uint16_t* C2 = g.C2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 64 + i * 16 + s;
    if (row >= mlim) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + 4 * gq;
      if (col >= g.N) continue;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q];
      const int64_t o = (int64_t)row * g.ldc + col;
      if constexpr (EPI == 1) {
        const uint2 dm = *reinterpret_cast<const uint2*>(g.Dmul + o);
        v[0] *= bf16_lo(dm.x);
        v[1] *= bf16_hi(dm.x);
        v[2] *= bf16_lo(dm.y);
        v[3] *= bf16_hi(dm.y);
      }
      uint2 out;
      if constexpr (EPI == 2) {
        uint2 d2;
        d2.x = pack_bf16x2(activation_grad<ACT>(v[0]), activation_grad<ACT>(v[1]));
        d2.y = pack_bf16x2(activation_grad<ACT>(v[2]), activation_grad<ACT>(v[3]));
        *reinterpret_cast<uint2*>(C2 + o) = d2;
        out.x = pack_bf16x2(activation_bf16<ACT>(v[0]), activation_bf16<ACT>(v[1]));
        out.y = pack_bf16x2(activation_bf16<ACT>(v[2]), activation_bf16<ACT>(v[3]));
      } else {
        out.x = pack_bf16x2(v[0], v[1]);
        out.y = pack_bf16x2(v[2], v[3]);
      }
      *reinterpret_cast<uint2*>(C + o) = out;
    }
  }
}

// fp32 layers: the same products with plain loads, 64 x 64 tiles, BK = 16, 4 x 4
// outputs per thread.
template <bool A_KC, bool B_KC, bool SEGK, int EPI, int ACT>
__global__ __launch_bounds__(256) void bwd_gemm_f32_kernel(BwdGemmArgs g) {
  constexpr int TB = 64, TK = 16;
  __shared__ float sA[TK][TB + 4];
  __shared__ float sB[TK][TB + 4];
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* B = reinterpret_cast<const float*>(g.B);
  int e, row0, row_end, m0, n0, k_lo, k_hi;
  if constexpr (SEGK) {
    const int tiles = g.n_tiles_m * g.n_tiles_n;
    e = blockIdx.x / tiles;
    const int t = blockIdx.x - e * tiles;
    m0 = (t / g.n_tiles_n) * TB;
    n0 = (t % g.n_tiles_n) * TB;
    row0 = 0;
    row_end = g.M;
    k_lo = g.offsets[e];
    k_hi = g.offsets[e + 1];
  } else {
    const int mt = blockIdx.x / g.n_tiles_n;
    if (mt >= g.tile_start[g.E]) return;
    e = g.tile_start[g.E + 1 + mt];
    row0 = g.offsets[e] + (mt - g.tile_start[e]) * TB;
    row_end = g.offsets[e + 1];
    n0 = (blockIdx.x - mt * g.n_tiles_n) * TB;
    m0 = row0;
    k_lo = 0;
    k_hi = g.K;
  }
  const int mlim = SEGK ? g.M : row_end;
  const float* Be = B + (SEGK ? 0 : (int64_t)e * g.b_expert_stride);
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = k_lo; k0 < k_hi; k0 += TK) {
    for (int i = tid; i < TB * TK; i += 256) {
      const int r = i / TK, kk = i % TK;  // A tile element (row r, k kk)
      const int gm = m0 + r, gk = k0 + kk;
      float va = 0.0f;
      if (gm < mlim && gk < k_hi) va = A_KC ? A[(int64_t)gm * g.lda + gk] : A[(int64_t)gk * g.lda + gm];
      sA[kk][r] = va;
      const int gn = n0 + r;
      float vb = 0.0f;
      if (gn < g.N && gk < k_hi) vb = B_KC ? Be[(int64_t)gn * g.ldb + gk] : Be[(int64_t)gk * g.ldb + gn];
      sB[kk][r] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = reinterpret_cast<float*>(g.C) + (SEGK ? (int64_t)e * g.c_expert_stride : 0);
  float* C2 = reinterpret_cast<float*>(g.C2);
  const float* Dm = reinterpret_cast<const float*>(g.Dmul);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= mlim) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= g.N) continue;
      const int64_t o = (int64_t)row * g.ldc + col;
      float v = acc[i][j];
      if constexpr (EPI == 1) v *= Dm[o];
      if constexpr (EPI == 2) {
        C2[o] = activation_grad<ACT>(v);
        v = activation<ACT>(v);
      }
      C[o] = v;
    }
  }
}

template <bool A_KC, bool B_KC, bool SEGK, int EPI, int ACT>
hipError_t launch_one(const BwdGemmArgs& g, int64_t blocks, bool bf16, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL((bwd_gemm_bf16_kernel<A_KC, B_KC, SEGK, EPI, ACT>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, g);
  else
    hipLaunchKernelGGL((bwd_gemm_f32_kernel<A_KC, B_KC, SEGK, EPI, ACT>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_kind(BwdGemmKind kind, const BwdGemmArgs& g, int64_t blocks, bool bf16, hipStream_t s) {
  switch (kind) {
    case kBwdRecompute1: return launch_one<true, false, false, 2, ACT>(g, blocks, bf16, s);
    case kBwdRecompute2: return launch_one<true, false, false, 0, ACT>(g, blocks, bf16, s);
    case kBwdDataGrad2: return launch_one<true, true, false, 1, ACT>(g, blocks, bf16, s);
    case kBwdDataGrad1: return launch_one<true, true, false, 0, ACT>(g, blocks, bf16, s);
    default: return launch_one<false, false, true, 0, ACT>(g, blocks, bf16, s);  // weight gradients
  }
}

}  // namespace
}  // namespace moe

int bwd_gemm_tile_rows(int dtype) { return dtype == 1 ? moe::kBM : 64; }
int bwd_gemm_tile_cols(int dtype) { return dtype == 1 ? moe::kBN : 64; }

hipError_t launch_bwd_gemm(BwdGemmKind kind, const BwdGemmArgs& g, int64_t blocks, int dtype, int act,
                           hipStream_t s) {
  const bool bf16 = dtype == 1;
  return act == 0 ? moe::launch_kind<0>(kind, g, blocks, bf16, s) : moe::launch_kind<1>(kind, g, blocks, bf16, s);
}
