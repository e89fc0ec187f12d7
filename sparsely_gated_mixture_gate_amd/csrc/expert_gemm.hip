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
//   * tile map: a one-block kernel (in the forward path, the dispatch scan) turns
//     offsets[E+1] into the prefix of ceil(rows_e / BM) M-tiles per expert and a
//     table of the expert of every M-tile, so a GEMM block finds its tile with
//     two dependent loads and the host never synchronises on the ragged segment
//     sizes. The grid is an upper bound (ceil(R_max / BM) + E M-tiles); surplus
//     blocks exit at once.
//   * bf16 path: BM x BN x BK tiles, 512 threads = 2 x 4 waves of
//     (BM/2) x (BN/4), MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation. Tile
//     shape by the rows an expert can hold: capacity <= 160 -> 160 x 512 x 32
//     (layer 1, 3 stages) and 160 x 384 x 32 (layer 2, 4 stages), capacity <= 256
//     -> 256 x 256 x 32 (4 stages), both one M-tile per expert with 16-row MFMA
//     tiles past the segment skipped and their A rows loaded as zero; otherwise
//     about one tile of rows per expert -> 128 x 256 x 32 (3 stages, row tiles past
//     the segment skipped), large segments -> 256 x 256 x 64 (layer 1, 2 stages,
//     unswizzled activation rows: one 128-byte L2 request per row and k-tile) and
//     256 x 256 x 32 (layer 2, 4 stages). Where weights stream from HBM, wide
//     N-tiles re-read each expert's rows fewer times and read fewer LDS operand
//     bytes per weight byte (those reads compete with the weight loads). Both operands go
//     HBM -> LDS in their HBM layout by direct-to-LDS buffer loads (16-byte
//     chunks, XOR-swizzled per row against bank conflicts) into an NSTAGE-deep
//     ring, NSTAGE - 1 k-tiles in flight, explicit vmcnt waits and a fence-free
//     barrier. For the compute-bound shapes (256-row tiles) the main loop is
//     software-pipelined: the operands of the next 32-wide k unit are read from
//     LDS into a second register set between the MFMAs of the current one (one
//     read per two MFMAs, pinned with scheduling barriers), so the MFMA pipe does
//     not wait for LDS at each k-tile. Activation rows (K-contiguous) are read
//     with ds_read_b128, weight rows (N-contiguous) K-contiguous with the gfx950
//     transposing read ds_read_b64_tr_b16 (two per operand). The MFMA runs with swapped operands
//     (D = W^T A^T) so each lane ends with 4 consecutive output columns of a
//     row (8-byte stores); ReLU / GELU is applied in fp32 before the bf16
//     (nearest-even, v_cvt_pk_bf16_f32) store, GELU with a branch-free erf
//     accurate to 1.5e-7.
//   * scheduling: real tiles are dealt evenly to the 8 XCDs in contiguous
//     chunks (tiles sharing an activation or weight panel share that XCD's L2),
//     rastered inside each expert in groups of 4 M-tiles.
//   * fp32 path: a plain LDS-tiled fp32 FMA kernel (64x64x16 tiles).
#include <type_traits>

#include "common.h"
#include "lds_dma.h"



namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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
  if (e < E) {
    tile_start[e] = sc[e] - tiles;
    for (int j = 0; j < tiles; ++j) tile_start[E + 1 + sc[e] - tiles + j] = e;  // expert of each M-tile
  }
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

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kXcds = 8;     // MI355X: 8 XCDs, workgroups dealt round-robin, one L2 each
constexpr int kGroupM = 4;   // M-tiles per raster group inside an expert

// Chunk swizzles (16-byte chunks). A rows hold BK/8 chunks: physical =
// chunk ^ swz_a_rc(row) (below). B rows hold 32 chunks (256 bf16 of N):
// physical = chunk ^ 2*swz_b(k); swz_b spreads the 8 rows that one half-wave
// reads in a transposing load over 8 distinct 32-byte bank groups.
__device__ __forceinline__ int swz_b(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// Map this workgroup to (expert, M-tile rows, N-tile). Real tiles are spread
// evenly over the XCDs in contiguous chunks (tiles that share an activation
// panel or a weight panel then share an L2); inside an expert, tiles are
// rastered in groups of kGroupM M-tiles so a wave of workgroups covers a compact
// block of the output. Returns false for surplus workgroups.
__device__ __forceinline__ bool schedule_tile(const int32_t* __restrict__ tile_start,
                                              const int32_t* __restrict__ offsets, int E, int bm, int nt_count,
                                              int* e_out, int* row0, int* row_end, int* nt_out) {
  const int total = tile_start[E] * nt_count;
  const int per = (total + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  const int L = (b % kXcds) * per + slot;
  if (slot >= per || L >= total) return false;
  const int mt_lin = L / nt_count;
  const int lo = tile_start[E + 1 + mt_lin];  // the expert of M-tile mt_lin
  const int mt0 = tile_start[lo];
  const int mts = tile_start[lo + 1] - mt0;
  const int loc = L - mt0 * nt_count;
  const int group = loc / (kGroupM * nt_count);
  const int first = group * kGroupM;
  const int gm = min(kGroupM, mts - first);
  const int r = loc - group * kGroupM * nt_count;
  const int mt = first + r % gm;
  *nt_out = r / gm;
  *e_out = lo;
  *row0 = offsets[lo] + mt * bm;
  *row_end = offsets[lo + 1];
  return true;
}

// A rows of 64-wide k-tiles (8 chunks, 128 bytes) stay unswizzled: 8 lanes then load a
// row's 128 bytes in address order, which the vector L1 fetches as one request (a swizzled
// row costs two 64-byte requests, and the L1 keeps a bounded number in flight).
template <int RC>
__device__ __forceinline__ int swz_a_rc(int row) {
  if constexpr (RC == 8) {
    return 0;
  } else {
    return (row >> 2) & 3;
  }
}

// C[rows of segment e] = act?(A . W[e]); A [R][K], W [E][K][N], C [R][N], all bf16.
// BM x BN x BK tiles (BN = 256 or 128), NW waves (64 NW threads) of WNT
// columns each, (NW / (BN/WNT)) x (BN/WNT); NSTAGE-deep LDS ring fed by
// direct-to-LDS buffer loads (NSTAGE - 1 k-tiles in flight).
template <int BM, int BN, int BK, int NSTAGE, int ACT, bool APPLY_ACT, bool SKIP, int NW, int WNT, bool PF>
__global__ __launch_bounds__(64 * NW, (BM / (NW / (BN / WNT))) * WNT > 8192 ? 1 : 8 / NW) void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ W,
                                                                uint16_t* __restrict__ C,
                                                                const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ tile_start, int E,
                                                                int K, int N, int n_tiles_n,
                                                                const int32_t* __restrict__ a_map, int64_t a_rows,
                                                                const int32_t* __restrict__ c_map,
                                                                const float* __restrict__ c_scale) {
  // a_map (or null): A row r of a segment is row a_map[r] of the a_rows-row buffer A.
  // c_map (or null; layer 2 only): C row r is written to row c_map[r], scaled by c_scale[c_map[r]].
  constexpr int NT = 64 * NW;            // threads
  constexpr int WN_W = BN / WNT;         // waves along N
  constexpr int WM_W = NW / WN_W;        // waves along M
  constexpr int BCR = BN / 8;            // 16-byte chunks per B row
  constexpr int WM = BM / WM_W;          // wave tile rows
  constexpr int MI = WM / 16;            // 16-row MFMA tiles per wave
  constexpr int NI = WNT / 16;           // 16-column MFMA tiles per wave
  constexpr int RC = BK / 8;             // 16-byte chunks per A row
  constexpr int A_CH = BM * RC;          // chunks per A tile
  constexpr int B_CH = BK * BCR;         // chunks per B tile
  constexpr int A_LD = (A_CH + NT - 1) / NT;  // A loads per thread per tile (the last round may be partial)
  constexpr int A_TAIL_W = (A_CH % NT) / 64;  // waves that issue the partial last round (0: none)
  constexpr int B_LD = B_CH / NT;
  constexpr int LD_HI = A_LD + B_LD;                       // loads per tile of waves < A_TAIL_W
  constexpr int LD_LO = A_LD - (A_TAIL_W ? 1 : 0) + B_LD;  // loads per tile of the other waves
  constexpr int STAGE_CH = A_CH + B_CH;
  static_assert(A_CH % 64 == 0 && B_CH % NT == 0 && WN_W * WM_W == NW, "tile / thread mismatch");
  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "stages");
  static_assert((BN == 128 || BN == 256 || BN == 384 || BN == 512) && WM % 16 == 0 && WNT % 16 == 0, "tile shape");
  __shared__ uint4 smem[NSTAGE * STAGE_CH];

  int e, row0, row_end, nt;
  if (!schedule_tile(tile_start, offsets, E, BM, n_tiles_n, &e, &row0, &row_end, &nt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = nt * BN;
  const int nk = (K + BK - 1) / BK;
  const int k_last = (nk - 1) * BK;
  const bool k_tail = (K % BK) != 0;
  const int rows = row_end - row0;

  // Per-thread byte offsets, fixed for the whole K loop; the k-tile advances the
  // wave-uniform soffset. Lane l fills LDS slot l of its wave's 64-chunk run, so it
  // fetches the chunk that the XOR swizzle places in that slot. Rows past the
  // segment are clamped (read, never stored). In the last, partial k-tile the A
  // chunks past K are clamped inside the row (finite data) and the B rows past K
  // (and B columns past N throughout) point outside the buffer, which loads zero.
  // scattered output rows: their targets and scales are loaded now, so the loads
  // complete under the main loop
  int64_t orow_m[MI];
  float scale_m[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    orow_m[mi] = 0;
    scale_m[mi] = 1.0f;
  }
  if (!APPLY_ACT && c_map) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int grow = row0 + (wave / WN_W) * WM + mi * 16 + (tid & 15);
      if (grow < row_end) {
        orow_m[mi] = c_map[grow];
        scale_m[mi] = c_scale[orow_m[mi]];
      }
    }
  }
  const bool gather = a_map != nullptr;
  const int32x4 rsA = gather ? buffer_rsrc(A, (uint32_t)(a_rows * K * 2))
                             : buffer_rsrc(A + (int64_t)row0 * K, (uint32_t)rows * K * 2);
  const int32x4 rsB = buffer_rsrc(W + (int64_t)e * K * N, (uint32_t)K * N * 2);
  constexpr int kOut = 0x7FFFFFF0;  // byte offset past any operand (K*N*2 < 2^31 - 16 is checked on the host)
  int voffA[A_LD], voffA_last[A_LD], voffB[B_LD], voffB_last[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + NT * i;
    const int row = c / RC, phys = c % RC;
    const int kc = phys ^ swz_a_rc<RC>(row);
    const int lrow = min(row, rows - 1);
    // row of the A buffer (gathered rows: T * K * 2 < 2^32 is checked on the host)
    const uint32_t arow = gather ? (uint32_t)a_map[row0 + lrow] : (uint32_t)lrow;
    voffA[i] = (int)((arow * (uint32_t)K + (uint32_t)(kc * 8)) * 2u);
    voffA_last[i] = (int)((arow * (uint32_t)K + (uint32_t)min(kc * 8, K - k_last - 8)) * 2u);  // + soffset k_last*2
    // rows past the segment load zero (gathered: they repeat the last row; never stored either way)
    if (SKIP && row >= rows && !gather) voffA[i] = voffA_last[i] = kOut;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = tid + NT * i;
    const int kr = c / BCR, phys = c % BCR;
    const int nc = phys ^ (2 * swz_b(kr));
    const int gn = n0 + nc * 8;
    voffB[i] = gn < N ? (kr * N + gn) * 2 : kOut;
    voffB_last[i] = (gn < N && k_last + kr < K) ? (kr * N + gn) * 2 : kOut;
  }
  const uint32_t lds0 = lds_address(&smem[0]);

  auto issue = [&](int kt) {
    const int st = kt % NSTAGE;
    const bool last = k_tail && kt == nk - 1;
    const int soffA = kt * BK * 2;
    const int soffB = kt * BK * N * 2;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      if (A_TAIL_W && i == A_LD - 1 && wave >= A_TAIL_W) break;
      const uint32_t dst = lds0 + (uint32_t)((st * STAGE_CH + i * NT + wave * 64) * 16);
      load_to_lds(__builtin_amdgcn_readfirstlane(dst), last ? voffA_last[i] : voffA[i], rsA, soffA);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const uint32_t dst = lds0 + (uint32_t)((st * STAGE_CH + A_CH + i * NT + wave * 64) * 16);
      // SKIP shapes: most experts fit one M-tile, so their weight bytes are read by one
      // workgroup row only and are streamed past the caches
      if constexpr (SKIP)
        load_to_lds_nt(__builtin_amdgcn_readfirstlane(dst), last ? voffB_last[i] : voffB[i], rsB, soffB);
      else
        load_to_lds(__builtin_amdgcn_readfirstlane(dst), last ? voffB_last[i] : voffB[i], rsB, soffB);
    }
  };

  const int wm = wave / WN_W, wn = wave % WN_W;
  // 16-row MFMA tiles wholly past the segment are neither read nor multiplied (SKIP
  // shapes; and in the pipelined loop, the last, partial M-tile of each expert)
  const int mact = (SKIP || PF) ? __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * WM + 15) / 16))) : MI;
  const int g = lane >> 4;   // k-group of 8 inside a 32-wide k step
  const int s = lane & 15;
  floatx4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // A operand (16 rows x 8 k of a 32-wide k step) of MFMA row tile mi from stage st
  typedef __attribute__((address_space(3))) char lds_char;
  auto rd_a = [&](int st, int ks, int mi) -> bf16x8 {
    const uint4* sA = &smem[st * STAGE_CH];
    const int row = wm * WM + mi * 16 + s;
    const int ch = ks * 4 + g;
    return __builtin_bit_cast(bf16x8, sA[row * RC + (ch ^ swz_a_rc<RC>(row))]);
  };
  // B operand of MFMA column tile ni. Transposing LDS read: source lane s of each
  // 16-lane group points at row k0 + s/4, columns n + 4*(s%4) .. +3; lane L of the
  // group then receives W[k0 .. k0+3][n + L]. Two reads give the 8 k-values.
  auto rd_b = [&](int st, int ks, int ni) -> bf16x8 {
    lds_char* sB = (lds_char*)(&smem[st * STAGE_CH + A_CH]);
    const int krow = ks * 32 + 8 * g + (s >> 2);
    const int ncol = wn * WNT + ni * 16 + 4 * (s & 3);
    const int c = ncol >> 3;
    const int b0 = krow * (BN * 2) + ((c ^ (2 * swz_b(krow))) << 4) + ((ncol & 7) << 1);
    const int b1 = (krow + 4) * (BN * 2) + ((c ^ (2 * swz_b(krow + 4))) << 4) + ((ncol & 7) << 1);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sB + b0));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(sB + b1));
    const short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  };
  // all MFMAs of k-tile st, operands read just before use
  auto compute = [&](int st) {
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        if (mi < mact) af[mi] = rd_a(st, ks, mi);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = rd_b(st, ks, ni);
      // swapped operands: D[n][m] = sum_k W[k][n] A[m][k], so each lane ends with
      // 4 consecutive output columns of one row
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= mact) break;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  // Software pipeline over 32-wide k units: the operands of unit u + 1 are read
  // from LDS into the second register set while the MFMAs of unit u run. A
  // barrier precedes the first read of each k-tile; before it every wave has
  // finished its reads of the previous k-tile, whose stage is then refilled.
  // DYN: this wave multiplies only its first mact 16-row tiles (a partial M-tile,
  // or the SKIP shapes); full tiles keep a fixed, pinned instruction schedule.
  auto pipelined = [&](auto dyn_c) {
    constexpr bool DYN = decltype(dyn_c)::value;
    constexpr int KS = BK / 32;
    constexpr int Q = MI * NI;   // MFMAs per unit
    constexpr int NR = NI + MI;  // operand reads per unit (a B operand = two transposing reads)
    bf16x8 fa[2][MI], fb[2][NI];
    // MFMAs of the unit in set CUR, with the reads of unit (nst, nks) into the other set
    // spread evenly over them (B operands first: every MFMA of a row tile needs all of them).
    auto unit = [&](auto cur_c, int nst, int nks) {
      constexpr int CUR = decltype(cur_c)::value, NXT = CUR ^ 1;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int mi = q / NI, ni = q % NI;
        if (!DYN || mi < mact)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[CUR][ni], fa[CUR][mi], acc[mi][ni], 0, 0, 0);
        if constexpr (!DYN) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // this MFMA, then its reads
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          if ((r * Q) / NR != q) continue;
          if (r < NI) {
            fb[NXT][r] = rd_b(nst, nks, r);
            if constexpr (!DYN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          } else if (!DYN || r - NI < mact) {
            fa[NXT][r - NI] = rd_a(nst, nks, r - NI);
            if constexpr (!DYN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
      }
    };
    auto wait_tile = [&](auto maxrem_c, int rem) {
      constexpr int MR = decltype(maxrem_c)::value;
      if (A_TAIL_W == 0 || wave < A_TAIL_W) wait_tiles<LD_HI, MR>(rem);
      else wait_tiles<LD_LO, MR>(rem);
    };
#pragma unroll
    for (int t = 0; t < NSTAGE; ++t)
      if (t < nk) issue(t);
    wait_tile(std::integral_constant<int, NSTAGE - 1>{}, min(NSTAGE - 1, nk - 1));
    block_barrier();
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) fb[0][ni] = rd_b(0, 0, ni);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      if (!DYN || mi < mact) fa[0][mi] = rd_a(0, 0, mi);
    const int nu = nk * KS;
    // one unit: u = kt * KS + ks, register set u & 1
    auto step = [&](auto cur_c, int u) {
      const int kt = u / KS, ks = u - kt * KS;
      int nst = kt % NSTAGE, nks = ks + 1;
      if (nks == KS) {
        nks = 0;
        if (kt + 1 < nk) {
          wait_lgkm0();
          wait_tile(std::integral_constant<int, NSTAGE - 2>{}, min(NSTAGE - 2, nk - 2 - kt));
          block_barrier();  // tile kt + 1 is in LDS; every wave is done with tile kt
          if (kt + NSTAGE < nk) issue(kt + NSTAGE);
          nst = (kt + 1) % NSTAGE;
        }
      }
      unit(cur_c, nst, nks);
    };
    for (int u = 0; u < nu; u += 2) {
      step(std::integral_constant<int, 0>{}, u);
      if (u + 1 < nu) step(std::integral_constant<int, 1>{}, u + 1);
    }
  };
  if constexpr (PF) {
    if (SKIP || mact < MI) pipelined(std::true_type{});
    else pipelined(std::false_type{});
  }
  if constexpr (!PF) {
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
      if (t < nk) issue(t);
    for (int kt = 0; kt < nk; ++kt) {
      if (A_TAIL_W == 0 || wave < A_TAIL_W)
        wait_tiles<LD_HI, NSTAGE - 2>(min(NSTAGE - 2, nk - 1 - kt));
      else
        wait_tiles<LD_LO, NSTAGE - 2>(min(NSTAGE - 2, nk - 1 - kt));
      block_barrier();  // tile kt is in LDS for every wave; buffer of tile kt-1 is free
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1);
      compute(kt % NSTAGE);
    }
  }

  // epilogue: lane holds C[m = .. + s][n = .. + 4g + j], j = 0..3, per MFMA tile
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int grow = row0 + wm * WM + mi * 16 + s;
    if (grow >= row_end) continue;
    const int64_t orow = (!APPLY_ACT && c_map) ? orow_m[mi] : grow;
    const float scale = scale_m[mi];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int gcol = n0 + wn * WNT + ni * 16 + 4 * g;
      if (gcol >= N) continue;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // layer 1 never scatters; in layer 2 the scale is 1 unless rows are scattered
        if constexpr (APPLY_ACT) v[j] = activation_bf16<ACT>(acc[mi][ni][j]);
        else v[j] = scale * acc[mi][ni][j];
      }
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(C + orow * N + gcol) = o;
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

// Grid rounded up to a multiple of the XCD count (surplus workgroups exit at once).
dim3 grid_for(int64_t tiles) { return dim3((unsigned)(((tiles + kXcds - 1) / kXcds) * kXcds)); }

// PF: the software-pipelined main loop (operands of the next 32-wide k unit read
// during the MFMAs of the current one), for the compute-bound tile shapes.
// BK, NSTAGE, BN, WNT: layer 2 (and layer 1 unless BK1 .. WNT1 are given).
template <int BM, int BK, int NSTAGE, int ACT, bool SKIP, bool PF, int NW = 8, int WNT = 64, int BN = 256,
          int BK1 = BK, int NSTAGE1 = NSTAGE, int BN1 = BN, int WNT1 = WNT>
hipError_t launch_bf16(const FfnLaunch& a, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (!a.tile_map_ready) {
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, BM, a.tile_start);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t mtiles = (a.max_rows + BM - 1) / BM + a.E;
  const int nt1 = (a.f + BN1 - 1) / BN1, nt2 = (a.d + BN - 1) / BN;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN1, BK1, NSTAGE1, ACT, true, SKIP, NW, WNT1, PF>), grid_for(mtiles * nt1),
                     dim3(64 * NW), 0, s, static_cast<const uint16_t*>(a.x_src ? a.x_src : a.x_perm),
                     static_cast<const uint16_t*>(a.w1), static_cast<uint16_t*>(a.h1), a.offsets, a.tile_start, a.E,
                     a.d, a.f, nt1, a.x_src ? a.row_src : nullptr, a.T, nullptr, nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.mid_event && (err = hipEventRecord(static_cast<hipEvent_t>(a.mid_event), s)) != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, BK, NSTAGE, ACT, false, SKIP, NW, WNT, PF>), grid_for(mtiles * nt2),
                     dim3(64 * NW), 0, s, static_cast<const uint16_t*>(a.h1), static_cast<const uint16_t*>(a.w2),
                     static_cast<uint16_t*>(a.y_out ? a.y_out : a.y_perm), a.offsets, a.tile_start, a.E, a.f, a.d, nt2,
                     nullptr, 0, a.y_out ? a.row_src : nullptr, a.y_out ? a.gate : nullptr);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_f32(const FfnLaunch& a, hipStream_t s) {
  constexpr int TB = 64;
  hipError_t err = hipSuccess;
  if (!a.tile_map_ready) {
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, TB, a.tile_start);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t mtiles = (a.max_rows + TB - 1) / TB + a.E;
  const int nt1 = (a.f + TB - 1) / TB, nt2 = (a.d + TB - 1) / TB;
  hipLaunchKernelGGL((grouped_gemm_f32_kernel<ACT, true>), dim3((unsigned)(mtiles * nt1)), dim3(256), 0, s,
                     static_cast<const float*>(a.x_perm), static_cast<const float*>(a.w1),
                     static_cast<float*>(a.h1), a.offsets, a.tile_start, a.E, a.d, a.f, nt1);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.mid_event && (err = hipEventRecord(static_cast<hipEvent_t>(a.mid_event), s)) != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_gemm_f32_kernel<ACT, false>), dim3((unsigned)(mtiles * nt2)), dim3(256), 0, s,
                     static_cast<const float*>(a.h1), static_cast<const float*>(a.w2),
                     static_cast<float*>(a.y_perm), a.offsets, a.tile_start, a.E, a.f, a.d, nt2);
  return hipGetLastError();
}

// Tile configuration of a layer, from what the host knows: the dtype, the
// capacity and the expected rows per expert.
enum FfnTiles { kTilesF32, kTiles160Skip, kTiles256Skip, kTiles256, kTiles128 };
FfnTiles ffn_tiles(int dtype, int64_t capacity, int64_t max_rows, int E) {
  if (dtype != 1) return kTilesF32;
  // A capacity of at most 160 (256) rows puts every expert in one 160-row
  // (256-row) M-tile, so each weight panel is streamed once; MFMA tiles past the
  // segment are skipped.
  if (capacity >= 0 && capacity <= 160) return kTiles160Skip;
  if (capacity >= 0 && capacity <= 256) return kTiles256Skip;
  // Otherwise the expected rows per expert decide the M tile: weight-streaming
  // experts (about one tile of rows each) take 128-row tiles, large segments 256.
  return max_rows / E >= 512 ? kTiles256 : kTiles128;
}

template <int ACT>
hipError_t launch_ffn_act(const FfnLaunch& a, hipStream_t s) {
  switch (ffn_tiles(a.dtype, a.capacity, a.max_rows, a.E)) {
    case kTilesF32: return launch_f32<ACT>(a, s);
    // weight-streaming, one M-tile per expert: wide N-tiles (fewer re-reads of each
    // expert's rows, fewer LDS operand reads per weight byte): layer 1 512 columns,
    // layer 2 384 columns (two tiles of a 768-wide output)
    case kTiles160Skip: return launch_bf16<160, 32, 4, ACT, true, false, 8, 96, 384, 32, 3, 512, 128>(a, s);
    case kTiles256Skip: return launch_bf16<256, 32, 4, ACT, true, true>(a, s);
    // layer 1 (K = d_model, the shorter) in 64-wide k-tiles, 2 stages: one 128-byte request per
    // activation row and k-tile instead of two (2.39 -> 2.28 ms at dropless_top1); layer 2
    // keeps 32-wide k-tiles in 4 stages (two 64 KB stages left its long K 27% slower)
    case kTiles256: return launch_bf16<256, 32, 4, ACT, false, true, 8, 128, 256, 64, 2, 256, 128>(a, s);
    // about one M-tile of rows per expert, no capacity: 256-column tiles on both layers
    // (twice the tiles of 512-column ones, so the tile rounds of a skewed routing stay
    // fuller: layer 2 of noisy_top4 has ~320 M-tiles for 256 CUs); most segments fill
    // part of their one tile, so MFMA row tiles past the segment are skipped and the
    // weight panels are streamed with the non-temporal hint
    default: return launch_bf16<128, 32, 3, ACT, true, false, 8, 64, 256>(a, s);
  }
}

}  // namespace
}  // namespace moe

int ffn_tile_rows(int dtype, int64_t capacity, int64_t max_rows, int E) {
  using namespace moe;
  switch (ffn_tiles(dtype, capacity, max_rows, E)) {
    case kTilesF32: return 64;
    case kTiles160Skip: return 160;
    case kTiles128: return 128;
    default: return 256;
  }
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* tile_start, hipStream_t s) {
  hipLaunchKernelGGL(moe::tile_map_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm, tile_start);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const FfnLaunch& a, hipStream_t s) {
  if (a.max_rows <= 0) return hipSuccess;
  return a.act == 0 ? moe::launch_ffn_act<0>(a, s) : moe::launch_ffn_act<1>(a, s);
}
