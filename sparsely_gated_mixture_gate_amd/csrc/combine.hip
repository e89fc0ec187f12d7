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

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const int32_t* __restrict__ slot_dest,
                                                      const float* __restrict__ gate, int64_t T, int k,
                                                      int chunks_per_row, uint4* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = i / chunks_per_row;
  if (t >= T) return;
  const int64_t c = i - t * chunks_per_row;
  constexpr int V = BF16 ? 8 : 4;
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.0f;
  for (int s = 0; s < k; ++s) {
    const int32_t slot = slot_dest[t * k + s];
    if (slot < 0) continue;
    const float g = gate[t * k + s];
    const uint4 v = load_nt(yp + (int64_t)slot * chunks_per_row + c);
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
  if (a.dtype == 1) {
    hipLaunchKernelGGL(moe::combine_kernel<true>, grid, dim3(256), 0, s, static_cast<const uint4*>(a.y_perm),
                       a.slot_dest, a.topk_gate, a.T, a.k, cpr, static_cast<uint4*>(a.y));
  } else {
    hipLaunchKernelGGL(moe::combine_kernel<false>, grid, dim3(256), 0, s, static_cast<const uint4*>(a.y_perm),
                       a.slot_dest, a.topk_gate, a.T, a.k, cpr, static_cast<uint4*>(a.y));
  }
  return hipGetLastError();
}
