// expert_gemm.hip -- every expert's two-layer FFN over its contiguous segment
// of the expert-sorted rows, as two grouped GEMMs.
//
// Method: Shazeer et al. summary page (abstract, "Methode"): the experts are
// feed-forward sub-networks and each token is evaluated only by the experts it
// was routed to. "Problem und Motivation" names the shrinking-batch problem and
// GPUs' preference for uniform arithmetic: here every expert's rows, gathered
// from the whole batch, run as dense matrix tiles of one launch.
//   H1[r] = act(Xp[r] . W1[e]),  Yp[r] = H1[r] . W2[e]   for r in segment e.
//
// Design (gfx950):
//   * tile map: a one-block kernel turns offsets[E+1] into the prefix of
//     ceil(rows_e / BM) M-tiles per expert; GEMM blocks binary-search it, so the
//     host never synchronises on the ragged segment sizes. The grid is an upper
//     bound (ceil(R_max / BM) + E M-tiles); surplus blocks exit at once.
//   * bf16 path: 128x128x64 block tiles, 256 threads = 2x2 waves of 64x64, MFMA
//     v_mfma_f32_16x16x32_bf16 with fp32 accumulation. A (activations, K
//     contiguous) is copied to LDS in 16-byte chunks; B (weights [K][N], N
//     contiguous) is loaded as 8x8 bf16 blocks and transposed in registers so
//     both operands sit K-contiguous in LDS and each MFMA operand is one
//     ds_read_b128. Rows of 8 chunks are XOR-swizzled (chunk ^ (row ^ row>>3) & 7)
//     so fragment reads and tile writes are free of bank conflicts. Double-
//     buffered LDS with global loads for tile k+1 in flight during the MFMAs of
//     tile k. MFMA column c of N-subtile j of a wave maps to output column
//     4c + j, so each lane ends with 4 consecutive columns per row and stores
//     8 bytes; the activation (ReLU / exact GELU) is applied in fp32 before the
//     bf16 (nearest-even) store.
//   * fp32 path: a plain LDS-tiled fp32 FMA kernel (64x64x16 tiles).
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;

__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                        int32_t* __restrict__ tile_start) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  const int32_t tiles = e < E ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
  sc[e] = tiles;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) tile_start[e] = sc[e] - tiles;
  if (e == E - 1) tile_start[E] = sc[e];
}

// Locate the expert and row range of M-tile mt. Returns false past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ tile_start, const int32_t* __restrict__ offsets,
                                          int E, int mt, int bm, int* e_out, int* row0, int* row_end) {
  if (mt >= tile_start[E]) return false;
  int lo = 0, hi = E;  // invariant: tile_start[lo] <= mt < tile_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  *e_out = lo;
  *row0 = offsets[lo] + (mt - tile_start[lo]) * bm;
  *row_end = offsets[lo + 1];
  return true;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// C[rows of segment e] = act?(A . W[e]); A [R][K], W [E][K][N], C [R][N], all bf16.
template <int ACT, bool APPLY_ACT>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ W,
                                                                   uint16_t* __restrict__ C,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ tile_start, int E,
                                                                   int K, int N, int n_tiles_n) {
  __shared__ uint4 sA[2][BM * 8];
  __shared__ uint4 sB[2][BN * 8];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x / n_tiles_n;
  const int nt = blockIdx.x - mt * n_tiles_n;
  int e, row0, row_end;
  if (!find_tile(tile_start, offsets, E, mt, BM, &e, &row0, &row_end)) return;
  const int n0 = nt * BN;
  const uint16_t* __restrict__ We = W + (int64_t)e * K * N;

  // global -> register staging
  uint4 ra[4];
  uint4 rb[8];
  const bool b_loader = tid < 128;
  const int b_kb = tid >> 4, b_nb = tid & 15;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      int grow = row0 + row;
      grow = grow < row_end ? grow : row_end - 1;
      const int gk = k0 + kc * 8;
      ra[i] = gk < K ? *reinterpret_cast<const uint4*>(A + (int64_t)grow * K + gk) : make_uint4(0, 0, 0, 0);
    }
    if (b_loader) {
      const int gn = n0 + b_nb * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int gk = k0 + b_kb * 8 + r;
        rb[r] = (gk < K && gn < N) ? *reinterpret_cast<const uint4*>(We + (int64_t)gk * N + gn)
                                   : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      sA[buf][row * 8 + (kc ^ swz(row))] = ra[i];
    }
    if (b_loader) {
      // rb[r] holds k = 8*b_kb + r, n = 8*b_nb .. +7 (two per dword, low half = even n).
      // Output row n (= 8*b_nb + i) needs k = 8*b_kb .. +7 (two per dword, low half = even k).
      const uint32_t* w = reinterpret_cast<const uint32_t*>(rb);  // w[4*r + q]: k=r, n=2q,2q+1
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i >> 1;
        const bool hi = i & 1;
        uint4 o;
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo_k = w[4 * (2 * p) + q];
          const uint32_t hi_k = w[4 * (2 * p + 1) + q];
          d[p] = hi ? ((lo_k >> 16) | (hi_k & 0xFFFF0000u)) : ((lo_k & 0xFFFFu) | (hi_k << 16));
        }
        o.x = d[0]; o.y = d[1]; o.z = d[2]; o.w = d[3];
        const int row = b_nb * 8 + i;
        sB[buf][row * 8 + (b_kb ^ swz(row))] = o;
      }
    }
  };

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 64 + mi * 16 + (lane & 15);
        af[mi] = __builtin_bit_cast(bf16x8, sA[buf][row * 8 + (ch ^ swz(row))]);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int nrow = wn * 64 + (lane & 15) * 4 + ni;
        bfr[ni] = __builtin_bit_cast(bf16x8, sB[buf][nrow * 8 + (ch ^ swz(nrow))]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane>>4)+j of each 16-row subtile and columns
  // 4*(lane&15) + ni (ni = 0..3) of the wave's 64 columns.
  const int gcol = n0 + wn * 64 + (lane & 15) * 4;
  if (gcol >= N) return;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int grow = row0 + wm * 64 + mi * 16 + (lane >> 4) * 4 + j;
      if (grow >= row_end) continue;
      float v[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) v[ni] = APPLY_ACT ? activation<ACT>(acc[mi][ni][j]) : acc[mi][ni][j];
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(C + (int64_t)grow * N + gcol) = o;
    }
  }
}

// fp32 path: 64x64 tiles, BK = 16, each thread a 4x4 micro-tile.
template <int ACT, bool APPLY_ACT>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                               const float* __restrict__ W, float* __restrict__ C,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ tile_start, int E, int K,
                                                               int N, int n_tiles_n) {
  constexpr int TB = 64, TK = 16;
  __shared__ float sA[TK][TB + 4];
  __shared__ float sB[TK][TB + 4];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x / n_tiles_n;
  const int nt = blockIdx.x - mt * n_tiles_n;
  int e, row0, row_end;
  if (!find_tile(tile_start, offsets, E, mt, TB, &e, &row0, &row_end)) return;
  const int n0 = nt * TB;
  const float* __restrict__ We = W + (int64_t)e * K * N;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int i = tid; i < TB * TK; i += 256) {
      const int r = i / TK, kk = i % TK;
      int grow = row0 + r;
      grow = grow < row_end ? grow : row_end - 1;
      const int gk = k0 + kk;
      sA[kk][r] = gk < K ? A[(int64_t)grow * K + gk] : 0.0f;
      const int kb = i / TB, n = i % TB;
      const int gkb = k0 + kb, gn = n0 + n;
      sB[kb][n] = (gkb < K && gn < N) ? We[(int64_t)gkb * N + gn] : 0.0f;
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = row0 + ty * 4 + i;
    if (grow >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < N) C[(int64_t)grow * N + gn] = APPLY_ACT ? activation<ACT>(acc[i][j]) : acc[i][j];
    }
  }
}

template <int ACT>
hipError_t launch_ffn_act(const FfnLaunch& a, hipStream_t s) {
  const int bm = a.dtype == 1 ? BM : 64;
  const int bn = a.dtype == 1 ? BN : 64;
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, bm, a.tile_start);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t mtiles = (a.max_rows + bm - 1) / bm + a.E;
  const int nt1 = (a.f + bn - 1) / bn, nt2 = (a.d + bn - 1) / bn;
  if (a.dtype == 1) {
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<ACT, true>), dim3((unsigned)(mtiles * nt1)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.x_perm), static_cast<const uint16_t*>(a.w1),
                       static_cast<uint16_t*>(a.h1), a.offsets, a.tile_start, a.E, a.d, a.f, nt1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<ACT, false>), dim3((unsigned)(mtiles * nt2)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.h1), static_cast<const uint16_t*>(a.w2),
                       static_cast<uint16_t*>(a.y_perm), a.offsets, a.tile_start, a.E, a.f, a.d, nt2);
  } else {
    hipLaunchKernelGGL((grouped_gemm_f32_kernel<ACT, true>), dim3((unsigned)(mtiles * nt1)), dim3(256), 0, s,
                       static_cast<const float*>(a.x_perm), static_cast<const float*>(a.w1),
                       static_cast<float*>(a.h1), a.offsets, a.tile_start, a.E, a.d, a.f, nt1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((grouped_gemm_f32_kernel<ACT, false>), dim3((unsigned)(mtiles * nt2)), dim3(256), 0, s,
                       static_cast<const float*>(a.h1), static_cast<const float*>(a.w2),
                       static_cast<float*>(a.y_perm), a.offsets, a.tile_start, a.E, a.f, a.d, nt2);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

hipError_t launch_expert_ffn(const FfnLaunch& a, hipStream_t s) {
  if (a.max_rows <= 0) return hipSuccess;
  return a.act == 0 ? moe::launch_ffn_act<0>(a, s) : moe::launch_ffn_act<1>(a, s);
}
