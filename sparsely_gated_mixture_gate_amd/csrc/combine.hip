// combine.hip -- gate-weighted sum of each token's expert outputs, back in
// token order.
//
// Method: Shazeer et al. summary page, "Methode": y = sum_i G(x)_i E_i(x);
// the "Switch Transformer" listing adds each expert's output back at its
// tokens. A dropped assignment (slot -1) contributes nothing; surviving gates
// are not rescaled; a token with every slot dropped gets a zero row.
//
// Design (gfx950): one thread per 16-byte chunk of an output row; it reads
// the token's k slots and gates (cached, shared by the row's threads),
// gathers the k expert-output chunks, accumulates in fp32 with fma in slot
// order and stores once. HBM-bound: 2d bytes read per kept assignment plus
// 2d bytes written per token (bf16). Expert-output rows are read once and the
// output written once, both with the non-temporal hint.
#include "common.h"
#include "stream_io.h"

namespace moe {
namespace {

// KC: k known at compile time (1, 2, 4: every slot's index, gate and row loads are
// issued before the sums), or 0 (any k, one slot after the other).
template <bool BF16, int KC>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const int32_t* __restrict__ slot_dest,
                                                      const float* __restrict__ gate, int64_t T, int k_rt,
                                                      int chunks_per_row, uint4* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = i / chunks_per_row;
  if (t >= T) return;
  const int64_t c = i - t * chunks_per_row;
  const int k = KC > 0 ? KC : k_rt;
  constexpr int V = BF16 ? 8 : 4;
  constexpr int NS = KC > 0 ? KC : 1;  // slots whose loads are in flight together
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.0f;
  for (int s0 = 0; s0 < k; s0 += NS) {
    int32_t slot[NS];
    float gs[NS];
    uint4 vs[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      slot[u] = slot_dest[t * k + s0 + u];
      gs[u] = gate[t * k + s0 + u];
    }
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (slot[u] >= 0) vs[u] = load_nt(yp + (int64_t)slot[u] * chunks_per_row + c);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (slot[u] < 0) continue;  // slot order: the sums add the slots in order
      const float g = gs[u];
      const uint4 v = vs[u];
      if constexpr (BF16) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(g, bf16_lo(w[q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(g, bf16_hi(w[q]), acc[2 * q + 1]);
        }
      } else {
        acc[0] = __builtin_fmaf(g, __uint_as_float(v.x), acc[0]);
        acc[1] = __builtin_fmaf(g, __uint_as_float(v.y), acc[1]);
        acc[2] = __builtin_fmaf(g, __uint_as_float(v.z), acc[2]);
        acc[3] = __builtin_fmaf(g, __uint_as_float(v.w), acc[3]);
      }
    }
  }
  uint4 o;
  if constexpr (BF16) {
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
  } else {
    o.x = __float_as_uint(acc[0]);
    o.y = __float_as_uint(acc[1]);
    o.z = __float_as_uint(acc[2]);
    o.w = __float_as_uint(acc[3]);
  }
  store_nt(y + i, o);
}

}  // namespace
}  // namespace moe

hipError_t launch_combine(const CombineLaunch& a, hipStream_t s) {
  const int elt = a.dtype == 1 ? 2 : 4;
  const int cpr = a.d * elt / 16;
  const int64_t total = a.T * cpr;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const uint4*>(a.y_perm), a.slot_dest, a.topk_gate, a.T,
                       a.k, cpr, static_cast<uint4*>(a.y));
  };
  if (a.dtype == 1) {
    if (a.k == 1) launch(moe::combine_kernel<true, 1>);
    else if (a.k == 2) launch(moe::combine_kernel<true, 2>);
    else if (a.k == 4) launch(moe::combine_kernel<true, 4>);
    else launch(moe::combine_kernel<true, 0>);
  } else {
    if (a.k == 1) launch(moe::combine_kernel<false, 1>);
    else if (a.k == 2) launch(moe::combine_kernel<false, 2>);
    else if (a.k == 4) launch(moe::combine_kernel<false, 4>);
    else launch(moe::combine_kernel<false, 0>);
  }
  return hipGetLastError();
}
