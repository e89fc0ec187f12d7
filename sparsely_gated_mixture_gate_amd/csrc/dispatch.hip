// dispatch.hip -- group the T*k assignments by expert, keep the first C of
// each expert in token order, and copy the kept token rows into one
// expert-sorted buffer.
//
// Method: the "Switch Transformer" page's listing gathers, for each expert,
// the tokens routed to it; the "moe paper models" table 2 lists capacity
// factors (a per-expert buffer size). Overflow is dropped in token order:
// walking tokens in order (slots in order within a token), each assignment
// takes the next rank of its expert and is kept iff rank < C.
//
// Drop order: token order as above, or (option) first-choice priority, where every
// token's first choice is ranked before any token's second choice ("moe paper
// models" table 2, GShard row: top-2 with a capacity); the kernels then walk the
// [T, k] tables slot-major, so ranks and rows follow (slot, token) order.
//
// Design (gfx950), up to four launches, all integer work exact and deterministic:
//   count   per 1024-assignment block, per-expert counts (LDS integer atomics);
//           in the forward path extra blocks also reduce the gate's per-block
//           partial sums (one expert per wave);
//   scan    one block: for each expert, exclusive prefix over blocks (the
//           block's base rank), kept = min(count, C), offsets = exclusive
//           prefix over experts, the expert FFN's tile map, the losses. Not
//           launched when blocks x experts <= 16384: then every rank block
//           derives its own base ranks and the offsets from the raw counts;
//   rank    per block: stable ranks inside each wave from 64-lane ballots on
//           the bits of the expert id (multisplit), per-wave running counts in
//           LDS, then base + earlier waves + in-wave rank -> slot or -1; top-1
//           forward path: zero the output rows of dropped tokens;
//   permute one 16-byte chunk per thread: x_perm[r] = x[row_src[r]], reads of
//           whole rows, fully coalesced writes (not needed by the bf16 forward
//           path, whose expert GEMM gathers its rows from x).
#include "common.h"
#include "stream_io.h"
#include "route_tail.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;  // assignments per block: 4 waves x 4 steps x 64 lanes

// Walk position w -> index of the assignment in the [T, k] tables. Token order
// (slot order within a token) walks the tables as stored; first-choice priority
// walks slot 0 of every token, then slot 1, ...
__device__ __forceinline__ int64_t walk_pos(int64_t w, const DispatchLaunch& a) {
  return a.slot_major ? (w % a.T) * a.k + w / a.T : w;
}
__device__ __forceinline__ int64_t walk_token(int64_t w, const DispatchLaunch& a) {
  return a.slot_major ? w % a.T : w / a.k;
}

// Blocks [0, nb): per-block expert histograms. Blocks past nb (forward path): the
// routing step's per-expert sums, one expert per wave.
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int64_t n, int E,
                                                             int nb, int32_t* __restrict__ blk_cnt,
                                                             const DispatchLaunch tl) {
  if ((int)blockIdx.x >= nb) {
    const int e = ((int)blockIdx.x - nb) * 4 + (threadIdx.x >> 6);
    if (e < E)
      tail::reduce_expert(e, threadIdx.x & 63, tl.part_prob, tl.part_imp, tl.part_load, tl.part_cnt, tl.route_nblk,
                          E, tl.counts_routed, tl.red);
    return;
  }
  extern __shared__ int hist[];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  int eid[kChunk / 256];  // all loads in flight before the histogram updates
#pragma unroll
  for (int q = 0; q < kChunk / 256; ++q) {
    const int64_t a = base + q * 256 + threadIdx.x;
    eid[q] = a < n ? idx[walk_pos(a, tl)] : -1;
  }
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kChunk / 256; ++q)
    if (eid[q] >= 0) atomicAdd(&hist[eid[q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_cnt[(int64_t)e * nb + blockIdx.x] = hist[e];
}

// Inclusive prefix sum over the 1024 threads of the block (shuffles inside each
// wave, then the wave totals); sw holds 16 values.
__device__ int64_t block_incl_scan(int64_t v, int64_t* sw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) sw[wave] = v;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wave; ++w) base += sw[w];
  __syncthreads();  // sw is reused by the next scan
  return v + base;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ blk_cnt, int nb, int E,
                                                             int64_t C, int32_t* __restrict__ counts_kept,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_start, int tile_rows,
                                                             const int32_t* __restrict__ counts_routed,
                                                             const double* __restrict__ red, int64_t T, int k,
                                                             int noisy, float* __restrict__ aux_out) {
  __shared__ int64_t sw[16];
  __shared__ double sh[16];
  const int e = threadIdx.x;
  // inputs of the losses (forward path), loaded now so they arrive during the scans
  int32_t cr_e = 0;
  double r0 = 0.0, r1 = 0.0, r2 = 0.0;
  if (aux_out && e < E) {
    cr_e = counts_routed[e];
    r0 = red[e];
    r1 = red[E + e];
    r2 = red[2 * E + e];
  }
  // exclusive prefix of the block counts along expert e's row, 8 loads in flight
  int64_t run = 0;
  if (e < E) {
    int32_t* row = blk_cnt + (int64_t)e * nb;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = b0 + u < nb ? row[b0 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < nb) {
          row[b0 + u] = (int32_t)run;
          run += c[u];
        }
    }
  }
  const int64_t kept = (e < E) ? ((C >= 0 && run > C) ? C : run) : 0;
  if (e < E) counts_kept[e] = (int32_t)kept;
  const int64_t kept_incl = block_incl_scan(kept, sw);
  if (e < E) offsets[e] = (int32_t)(kept_incl - kept);
  if (e == E - 1) offsets[E] = (int32_t)kept_incl;
  if (tile_start) {
    // prefix of ceil(kept / tile_rows) M-tiles per expert for the expert FFN
    const int64_t tiles = (kept + tile_rows - 1) / tile_rows;
    const int64_t tiles_incl = block_incl_scan(tiles, sw);
    if (e < E) {
      const int32_t first = (int32_t)(tiles_incl - tiles);
      tile_start[e] = first;
      for (int64_t j = 0; j < tiles; ++j) tile_start[E + 1 + first + j] = e;  // expert of each M-tile
    }
    if (e == E - 1) tile_start[E] = (int32_t)tiles_incl;
  }
  // forward path: the balancing losses from the per-expert sums of the count kernel
  if (aux_out) tail::aux_from_values<1024>(e < E, cr_e, r0, r1, r2, E, T, k, noisy, aux_out, sh);
}

// SCAN = false: blk_base holds the exclusive prefixes of the block counts along
// each expert and offsets the segment starts (written by the scan kernel).
// SCAN = true (small count tables): blk_base holds the raw block counts; every
// rank block derives its own prefixes and the offsets from them, one extra block
// (blockIdx.x == nb, no ranks) writes counts_kept, offsets and the FFN tile map,
// and a second (nb + 1) the losses (as the scan kernel would), so no separate scan
// launch is needed and that work runs beside the ranks instead of before block 0's.
template <bool SCAN>
__global__ __launch_bounds__(256) void dispatch_rank_kernel(const int32_t* __restrict__ idx, int64_t n, int k,
                                                            int E, int nbits, int nb, int64_t C,
                                                            const int32_t* __restrict__ blk_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ slot_dest,
                                                            int32_t* __restrict__ row_src,
                                                            uint4* __restrict__ y_zero, int y_chunks,
                                                            const DispatchLaunch so) {
  extern __shared__ int wcnt[];  // [4 waves][E] running counts; SCAN: then base [E], segment starts [E + 1]
  // this thread's four expert ids, loaded first so that they arrive under the prefix work
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kChunk + wave * 256;
  int eid[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t a = base + q * 64 + lane;  // walk position
    eid[q] = (blockIdx.x < (unsigned)nb && a < n) ? idx[walk_pos(a, so)] : 0;
  }
  for (int i = threadIdx.x; i < 4 * E; i += 256) wcnt[i] = 0;
  int* const base_s = wcnt + 4 * E;
  int* const off_s = base_s + E;
  if constexpr (SCAN) {
    __shared__ int64_t sw[16];
    __shared__ double sh[16];
    if (blockIdx.x == nb + 1) {  // the second extra block: the losses, beside the other blocks
      if (so.route_tail && so.aux_out)
        tail::aux_block<256>(so.counts_routed, so.red, E, so.T, so.k, so.noisy, so.aux_out, sh);
      return;
    }
    // per expert: counts of the blocks before this one, and the total
    for (int e = threadIdx.x; e < E; e += 256) {
      const int32_t* row = blk_base + (int64_t)e * nb;
      int before = 0, tot = 0;
      for (int b0 = 0; b0 < nb; b0 += 16) {  // 16 loads in flight
        int32_t c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = b0 + u < nb ? row[b0 + u] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          before += b0 + u < (int)blockIdx.x ? c[u] : 0;
          tot += c[u];
        }
      }
      base_s[e] = before;
      off_s[e] = (C >= 0 && tot > C) ? (int)C : tot;  // kept rows, turned into segment starts below
    }
    __syncthreads();
    // segment starts: exclusive prefix of the kept rows over the experts (thread t: experts 4t .. 4t+3)
    int kept4[4];
    int64_t loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * (int)threadIdx.x + j;
      kept4[j] = e < E ? off_s[e] : 0;
      loc += kept4[j];
    }
    const int64_t incl = block_incl_scan(loc, sw);
    __syncthreads();
    int64_t run = incl - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * (int)threadIdx.x + j;
      if (e < E) off_s[e] = (int)run;
      run += kept4[j];
    }
    if (threadIdx.x == 255) off_s[E] = (int)incl;
    __syncthreads();
    if (blockIdx.x == nb) {  // the extra block: offsets, kept counts and tile map, no ranks
      for (int e = threadIdx.x; e <= E; e += 256) so.offsets[e] = off_s[e];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * (int)threadIdx.x + j;
        if (e < E) so.counts_kept[e] = kept4[j];
      }
      if (so.tile_start) {
        // prefix of ceil(kept / tile_rows) M-tiles per expert, and the expert of each M-tile
        int tiles4[4];
        int64_t tl = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tiles4[j] = (kept4[j] + so.tile_rows - 1) / so.tile_rows;
          tl += tiles4[j];
        }
        const int64_t tincl = block_incl_scan(tl, sw);
        int64_t first = tincl - tl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * (int)threadIdx.x + j;
          if (e < E) {
            so.tile_start[e] = (int32_t)first;
            for (int q = 0; q < tiles4[j]; ++q) so.tile_start[E + 1 + first + q] = e;
          }
          first += tiles4[j];
        }
        if (threadIdx.x == 255) so.tile_start[E] = (int32_t)tincl;
      }
      return;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ex[4], loc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t a = base + q * 64 + lane;  // walk position
    const bool valid = a < n;
    const int e = valid ? eid[q] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      same &= bit ? ones : ~ones;
    }
    const int before_in_wave = __popcll(same & lt_mask);
    const int prev = valid ? wcnt[wave * E + e] : 0;
    loc[q] = prev + before_in_wave;
    ex[q] = valid ? e : -1;
    __builtin_amdgcn_wave_barrier();
    if (valid && before_in_wave == 0) wcnt[wave * E + e] = prev + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  bool dropped[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = ex[q];
    dropped[q] = false;
    if (e < 0) continue;
    const int64_t a = base + q * 64 + lane;
    int64_t r = (SCAN ? (int64_t)base_s[e] : (int64_t)blk_base[(int64_t)e * nb + blockIdx.x]) + loc[q];
    for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
    const bool keep = C < 0 || r < C;
    const int32_t slot = keep ? (int32_t)((SCAN ? off_s[e] : offsets[e]) + r) : -1;
    slot_dest[walk_pos(a, so)] = slot;
    if (keep) row_src[slot] = (int32_t)walk_token(a, so);
    dropped[q] = !keep;
  }
  // top-1 layers: the output rows of dropped tokens are zero; the wave clears them
  // together, one row at a time, with coalesced 16-byte stores
  if (y_zero) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint64_t m = __ballot(dropped[q]);
      while (m) {
        const int j = __builtin_ctzll(m);
        m &= m - 1;
        uint4* yr = y_zero + (base + q * 64 + j) * y_chunks;  // k = 1: walk position = token
        for (int c = lane; c < y_chunks; c += 64) yr[c] = uint4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// x_perm[r, :] = x[row_src[r], :] for r < offsets[E]; 16-byte chunks.
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ row_src,
                                                           const int32_t* __restrict__ offsets, int E,
                                                           int chunks_per_row, int64_t total,
                                                           uint4* __restrict__ xp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t r = i / chunks_per_row;
  if (r >= offsets[E]) return;
  const int64_t c = i - r * chunks_per_row;
  store_nt(xp + i, load_nt(x + (int64_t)row_src[r] * chunks_per_row + c));  // each row streamed once
}

}  // namespace
}  // namespace moe

int64_t dispatch_num_blocks(int64_t assignments) { return (assignments + moe::kChunk - 1) / moe::kChunk; }

hipError_t launch_dispatch(const DispatchLaunch& a, hipStream_t s) {
  using namespace moe;
  const int64_t n = a.T * a.k;
  const int nb = (int)dispatch_num_blocks(n);
  hipError_t err;
  const int nred = a.route_tail ? (a.E + 3) / 4 : 0;  // blocks of the routing step's per-expert sums
  if (nb + nred > 0) {
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nb + nred), dim3(256), sizeof(int) * a.E, s, a.topk_idx, n, a.E,
                       nb, a.blk_cnt, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // small count tables: every rank block derives its own prefixes (no scan launch)
  const bool scan_in_rank = nb > 0 && (int64_t)nb * a.E <= 16384;
  if (!scan_in_rank) {
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, a.blk_cnt, nb, a.E, a.C, a.counts_kept,
                       a.offsets, a.tile_start, a.tile_rows, a.counts_routed, a.red, a.T, a.k, a.noisy,
                       a.route_tail ? a.aux_out : nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (nb == 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  const int y_chunks = a.d * (a.dtype == 1 ? 2 : 4) / 16;
  if (scan_in_rank) {
    // nb rank blocks and one block for offsets, tile map and losses, which then run side by side
    hipLaunchKernelGGL(dispatch_rank_kernel<true>, dim3(nb + 2), dim3(256), sizeof(int) * (6 * a.E + 1), s, a.topk_idx,
                       n, a.k, a.E, nbits, nb, a.C, a.blk_cnt, a.offsets, a.slot_dest, a.row_src,
                       static_cast<uint4*>(a.y_zero), y_chunks, a);
  } else {
    hipLaunchKernelGGL(dispatch_rank_kernel<false>, dim3(nb), dim3(256), sizeof(int) * 4 * a.E, s, a.topk_idx, n,
                       a.k, a.E, nbits, nb, a.C, a.blk_cnt, a.offsets, a.slot_dest, a.row_src,
                       static_cast<uint4*>(a.y_zero), y_chunks, a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int elt = a.dtype == 1 ? 2 : 4;
  const int cpr = a.d * elt / 16;
  const int64_t total = a.max_rows * cpr;
  if (total > 0 && !a.skip_permute) {
    hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint4*>(a.x), a.row_src, a.offsets, a.E, cpr, total,
                       static_cast<uint4*>(a.x_perm));
    err = hipGetLastError();
  }
  return err;
}
