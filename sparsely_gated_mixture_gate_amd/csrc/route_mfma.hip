// route_mfma.hip -- host side of the certified MFMA gate (route_mfma.h): the
// bf16 weight re-layout kernel and the launch of the gate kernel.
#include "route_mfma.h"

#include <atomic>

namespace moe {

extern template hipError_t launch_fused_kk<64, false>(int, const FusedArgs&, hipStream_t);
extern template hipError_t launch_fused_kk<64, true>(int, const FusedArgs&, hipStream_t);
extern template hipError_t launch_fused_kk<128, false>(int, const FusedArgs&, hipStream_t);
extern template hipError_t launch_fused_kk<128, true>(int, const FusedArgs&, hipStream_t);
extern template hipError_t launch_fused_kk<256, false>(int, const FusedArgs&, hipStream_t);
extern template hipError_t launch_fused_kk<256, true>(int, const FusedArgs&, hipStream_t);

namespace {

// bf16 weight copy [d][ncol]: gate only: column c = expert c; noisy: block q of
// 64 columns = gate columns of experts 32q .. 32q+31, then their noise columns.
// Zero past E. Noisy: also its transpose [ncol][d] after it (wt), so that the
// fallback gathers a candidate's gate and noise columns as contiguous rows.
__global__ __launch_bounds__(256) void route_wcat_kernel(const uint16_t* __restrict__ wg,
                                                         const uint16_t* __restrict__ wn,
                                                         uint16_t* __restrict__ wcat, uint16_t* __restrict__ wt,
                                                         int d, int E, int ncol) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * ncol) return;
  const int64_t j = i / ncol;
  const int c = (int)(i - j * ncol);
  const uint16_t* src = wg;
  int e = c;
  if (wn) {
    e = 32 * (c >> 6) + (c & 31);
    if (c & 32) src = wn;
  }
  const uint16_t v = e < E ? src[j * E + e] : (uint16_t)0;
  wcat[i] = v;
  if (wt) wt[(int64_t)c * d + j] = v;
}

int fused_ep(int E) { return E <= 64 ? 64 : (E <= 128 ? 128 : 256); }

}  // namespace
}  // namespace moe

bool route_fused_supported(int dtype, int E) { return dtype == 1 && E <= 256; }

size_t route_wcat_elems(int d, int E, bool noisy) {
  return (size_t)d * moe::fused_ep(E) * (noisy ? 4 : 1);  // noisy: [d][2 EP] and its transpose
}

// Tokens per block of the certified gate: a block holds most of a CU's LDS, so
// when 64-token blocks would leave CUs idle the blocks take 32 tokens. The CU
// count is cached per device in atomics (calls may come from several threads;
// every thread that fills an entry stores the same value).
int route_fused_tokens(int64_t T) {
  static std::atomic<int> cus_of[64];
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    cus = cus_of[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
      int n = 0;
      cus = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
      cus_of[dev].store(cus, std::memory_order_relaxed);
    }
  }
  return (T + 63) / 64 < cus ? 32 : 64;
}

hipError_t launch_route_fused(const RouteLaunch& a, bool noisy, int force_fallback, float* CL, float* SG, int lpad,
                              hipStream_t s) {
  using namespace moe;
  const int EP = fused_ep(a.E);
  const int ncol = EP * (noisy ? 2 : 1);
  const int64_t n = (int64_t)a.d * ncol;
  // a gate-only W_gate [d][E] with E = EP already is the weight layout the kernel reads
  const uint16_t* wcat = static_cast<const uint16_t*>(a.w_gate);
  if (noisy || a.E != EP) {
    hipLaunchKernelGGL(route_wcat_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.w_gate),
                       static_cast<const uint16_t*>(noisy ? a.w_noise : nullptr), a.wcat,
                       noisy ? a.wcat + (size_t)a.d * ncol : nullptr, a.d, a.E, ncol);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    wcat = a.wcat;
  }
  FusedArgs fa;
  fa.T = a.T;
  fa.d = a.d;
  fa.E = a.E;
  fa.k = a.k;
  fa.renormalize = a.renormalize;
  fa.tpb = route_fused_tokens(a.T);
  fa.nblk = (int)((a.T + fa.tpb - 1) / fa.tpb);
  fa.force_fallback = force_fallback;
  fa.lpad = lpad;
  fa.x = static_cast<const uint16_t*>(a.x);
  fa.wcat = wcat;
  fa.wt = noisy ? a.wcat + (size_t)a.d * ncol : nullptr;
  fa.bias = a.gate_bias;
  fa.noise = a.noise;
  fa.topk_idx = a.topk_idx;
  fa.topk_gate = a.topk_gate;
  fa.CL = CL;
  fa.SG = SG;
  fa.part_prob = a.part_prob;
  fa.part_imp = a.part_imp;
  fa.part_load = a.part_load;
  fa.part_cnt = a.part_cnt;
  fa.dbg = a.gate_mode == 3 ? a.logits_out : nullptr;
  const int kk = a.k + 1 < a.E ? a.k + 1 : a.E;
  if (EP == 64) return noisy ? launch_fused_kk<64, true>(kk, fa, s) : launch_fused_kk<64, false>(kk, fa, s);
  if (EP == 128) return noisy ? launch_fused_kk<128, true>(kk, fa, s) : launch_fused_kk<128, false>(kk, fa, s);
  return noisy ? launch_fused_kk<256, true>(kk, fa, s) : launch_fused_kk<256, false>(kk, fa, s);
}
