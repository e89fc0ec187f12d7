// moe_abi.hip -- the C ABI declared in include/moe.h: argument checks,
// workspace carve-up and the launch sequence of each entry point. Host code;
// no call here synchronises the stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "moe.h"
#include "common.h"

// Scratch of moe_dispatch_noalloc (the per-block expert counts of the dispatch):
// a fixed device array, one copy per GPU, held until the process ends. Host code
// never uses this name as an address: it looks up each device's copy with
// hipGetSymbolAddress (scratch_address below) and passes that pointer on.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

hipError_t launch_softplus(const float* z, float* out, int64_t n, hipStream_t s);
hipError_t launch_normal_noise(uint64_t seed, int64_t row0, int64_t rows, int cols, float* out, hipStream_t s);

namespace {

thread_local std::string g_last_error;

// Phase timing of moe_forward (moe_set_phase_events): caller-owned hipEvent_t handles.
constexpr int kPhaseEvents = 6;
thread_local void* g_phase_ev[kPhaseEvents] = {};

hipError_t record_phase(int i, hipStream_t s) {
  return g_phase_ev[i] ? hipEventRecord(static_cast<hipEvent_t>(g_phase_ev[i]), s) : hipSuccess;
}

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_params(const moe_params* p) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "params is NULL");
  if (p->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", (long long)p->T);
  if (p->E < 1) return fail(MOE_ERR_INVALID_ARG, "E = %d < 1", p->E);
  if (p->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 1024", p->E);
  if (p->k < 1 || p->k > p->E) return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, E=%d]", p->k, p->E);
  if (p->k > 8) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 8", p->k);
  if (p->d_model <= 0 || p->d_ff <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d_model = %d, d_ff = %d must be positive", p->d_model, p->d_ff);
  if (p->d_model % 8 || p->d_ff % 8)
    return fail(MOE_ERR_UNSUPPORTED, "d_model = %d and d_ff = %d must be multiples of 8", p->d_model, p->d_ff);
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype = %d", p->dtype);
  if (p->act != MOE_ACT_RELU && p->act != MOE_ACT_GELU) return fail(MOE_ERR_INVALID_ARG, "act = %d", p->act);
  if (p->renormalize != 0 && p->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "renormalize = %d (0 or 1)", p->renormalize);
  if (p->gate_mode < MOE_GATE_AUTO || p->gate_mode > MOE_GATE_EXPORT)
    return fail(MOE_ERR_INVALID_ARG, "gate_mode = %d (0, 1, 2 or 3)", p->gate_mode);
  if (p->T * (int64_t)p->k >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld >= 2^31", (long long)(p->T * p->k));
  if (isnan(p->capacity_factor)) return fail(MOE_ERR_INVALID_ARG, "capacity_factor is NaN");
  if (p->drop_order != MOE_DROP_TOKEN_ORDER && p->drop_order != MOE_DROP_FIRST_CHOICE)
    return fail(MOE_ERR_INVALID_ARG, "drop_order = %d (0 or 1)", p->drop_order);
  if (p->groups < 0 || p->k_group < 0)
    return fail(MOE_ERR_INVALID_ARG, "groups = %d and k_group = %d must be >= 0", p->groups, p->k_group);
  // 32-bit byte offsets inside one expert's weights and one row segment
  const int64_t elt = p->dtype == MOE_BF16 ? 2 : 4;
  const int64_t widest = p->d_model > p->d_ff ? p->d_model : p->d_ff;
  if ((int64_t)p->d_model * p->d_ff * elt >= (int64_t(1) << 31) - 16 ||
      p->T * (int64_t)p->k * widest * elt >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "an expert's weights or the permuted rows exceed 32-bit byte offsets");
  // 32-bit byte offsets inside the fp32 gate (+ noise) weights, column blocks of 128
  if ((int64_t)p->d_model * (2 * ((p->E + 63) / 64) * 64 + 128) * 4 >= (int64_t(1) << 31) - 16)
    return fail(MOE_ERR_UNSUPPORTED, "d_model * E too large for the gate weights' 32-bit byte offsets");
  return MOE_OK;
}

// Hierarchical layers: groups g >= 1 dividing E (E / g experts per group), k_group
// dividing k (k / k_group experts per kept group), k_group <= g, k / k_group <= E / g.
moe_status check_hier(const moe_params* p) {
  const int g = p->groups, kg = p->k_group;
  if (g < 1 || kg < 1) return fail(MOE_ERR_INVALID_ARG, "hierarchical layer needs groups >= 1 and k_group >= 1");
  if (p->E % g) return fail(MOE_ERR_INVALID_ARG, "E = %d is not a multiple of groups = %d", p->E, g);
  if (p->k % kg) return fail(MOE_ERR_INVALID_ARG, "k = %d is not a multiple of k_group = %d", p->k, kg);
  if (kg > g || p->k / kg > p->E / g)
    return fail(MOE_ERR_INVALID_ARG, "k_group = %d > groups = %d or k / k_group = %d > E / groups = %d", kg, g,
                p->k / kg, p->E / g);
  return MOE_OK;
}

// The flat gate's entry points take flat layers only.
moe_status check_flat(const moe_params* p) {
  if (p->groups > 1)
    return fail(MOE_ERR_INVALID_ARG, "groups = %d: a hierarchical layer's gate is moe_route_hier / moe_forward_hier",
                p->groups);
  return MOE_OK;
}

int64_t capacity_of(const moe_params* p) {
  if (p->capacity >= 0) return p->capacity;
  if (!(p->capacity_factor > 0.0)) return -1;
  return (int64_t)ceil(p->capacity_factor * (double)p->k * (double)p->T / (double)p->E);
}

int64_t max_rows_of(const moe_params* p) {
  const int64_t n = p->T * p->k;
  const int64_t C = capacity_of(p);
  if (C < 0) return n;
  const int64_t cap = C * p->E;
  return cap < n ? cap : n;
}

size_t elt_size(const moe_params* p) { return p->dtype == MOE_BF16 ? 2 : 4; }

// Sequential carve-up of a workspace into 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return r;
  }
};

struct RouteWs {
  float *wc, *lg;
  uint16_t* wcat;
  float *part_prob, *part_imp, *part_load;
  int32_t* part_cnt;
  double* red;
};
RouteWs carve_route(Carver& c, const moe_params* p, bool noisy) {
  const int64_t nblk = (p->T + 31) / 32;  // the most partial-sum blocks any gate path writes (32-token blocks)
  const size_t n = (size_t)p->E * (size_t)(nblk > 0 ? nblk : 1);
  RouteWs w;
  w.wc = c.take<float>(route_weight_floats(p->d_model, p->E, noisy));
  w.wcat = c.take<uint16_t>(route_wcat_elems(p->d_model, p->E, noisy));
  w.lg = c.take<float>(route_logit_floats(p->T, p->E, noisy));
  w.part_prob = c.take<float>(n);
  w.part_imp = c.take<float>(n);
  w.part_load = c.take<float>(n);
  w.part_cnt = c.take<int32_t>(n);
  w.red = c.take<double>(3 * (size_t)p->E);
  return w;
}

int32_t* carve_dispatch(Carver& c, const moe_params* p) {
  const int64_t nb = dispatch_num_blocks(p->T * p->k);
  return c.take<int32_t>((size_t)p->E * (size_t)(nb > 0 ? nb : 1));
}

struct FfnWs {
  int32_t* tile_start;
  void* h1;
};
FfnWs carve_ffn(Carver& c, const moe_params* p) {
  FfnWs w;
  // [E+1] M-tile prefix, then the expert of every M-tile (at most ceil(R / BM) + E tiles)
  const int64_t bm = ffn_tile_rows(p->dtype, capacity_of(p), max_rows_of(p), p->E);
  const int64_t mtiles = (max_rows_of(p) + bm - 1) / bm + p->E;
  w.tile_start = c.take<int32_t>((size_t)p->E + 1 + (size_t)mtiles);
  w.h1 = c.take<char>((size_t)max_rows_of(p) * (size_t)p->d_ff * elt_size(p));
  return w;
}

struct ForwardWs {
  RouteWs route;
  int32_t* blk_cnt;
  FfnWs ffn;
  int32_t *topk_idx, *counts_routed, *counts_kept, *offsets, *slot_dest, *row_src;
  float* topk_gate;
  void *x_perm, *y_perm;
};
ForwardWs carve_forward(Carver& c, const moe_params* p, bool noisy) {
  ForwardWs w;
  const size_t tk = (size_t)(p->T * p->k > 0 ? p->T * p->k : 1);
  const size_t rows = (size_t)(max_rows_of(p) > 0 ? max_rows_of(p) : 1);
  w.route = carve_route(c, p, noisy);
  w.blk_cnt = carve_dispatch(c, p);
  w.ffn = carve_ffn(c, p);
  w.topk_idx = c.take<int32_t>(tk);
  w.topk_gate = c.take<float>(tk);
  w.counts_routed = c.take<int32_t>((size_t)p->E);
  w.counts_kept = c.take<int32_t>((size_t)p->E);
  w.offsets = c.take<int32_t>((size_t)p->E + 1);
  w.slot_dest = c.take<int32_t>(tk);
  w.row_src = c.take<int32_t>(rows);
  // bf16: the expert GEMM gathers its rows from x (no x_perm) and, for top-1 layers,
  // writes y directly (no y_perm)
  const bool bf16 = p->dtype == MOE_BF16;
  w.x_perm = bf16 ? nullptr : c.take<char>(rows * (size_t)p->d_model * elt_size(p));
  w.y_perm = (bf16 && p->k == 1) ? nullptr : c.take<char>(rows * (size_t)p->d_model * elt_size(p));
  return w;
}

struct HierWs {
  float *wc_p, *lg_p, *wc_s, *lg_s;
  int32_t* order_p;
  float* gate_p;
  double* red;
};
HierWs carve_route_hier(Carver& c, const moe_params* p, bool noisy_p, bool noisy_s) {
  HierWs w;
  const int g = p->groups > 0 ? p->groups : 1, kg = p->k_group > 0 ? p->k_group : 1;
  const size_t T = (size_t)(p->T > 0 ? p->T : 1);
  w.wc_p = c.take<float>(route_weight_floats(p->d_model, g, noisy_p));
  w.lg_p = c.take<float>(route_logit_floats((int64_t)T, g, noisy_p));
  w.wc_s = c.take<float>(route_weight_floats(p->d_model, p->E, noisy_s));
  w.lg_s = c.take<float>(route_logit_floats((int64_t)T, p->E, noisy_s));
  w.order_p = c.take<int32_t>(T * (size_t)(kg + 1));
  w.gate_p = c.take<float>(T * (size_t)kg);
  w.red = c.take<double>((size_t)p->E + 2 * (size_t)g);
  return w;
}

struct ForwardHierWs {
  HierWs route;
  ForwardWs rest;  // its route part is unused
};

struct BackwardWs {
  RouteWs route;  // the canonical gate keeps H, clean logits and softplus values in route.lg
  int32_t* blk_cnt;
  int32_t* tile_start;
  int32_t *topk_idx, *counts_routed, *counts_kept, *offsets, *slot_dest, *row_src;
  float *topk_gate, *dg, *dimp, *dload, *dpsw, *dclean, *du, *part, *part_b;
  void *x_perm, *h1, *d1, *o, *dO;  // d1 holds act'(z), then dZ; o holds the outputs, then dXp
};
BackwardWs carve_backward(Carver& c, const moe_params* p, bool noisy) {
  BackwardWs w;
  const size_t tk = (size_t)(p->T * p->k > 0 ? p->T * p->k : 1);
  const size_t rows = (size_t)(max_rows_of(p) > 0 ? max_rows_of(p) : 1);
  const size_t te = (size_t)(p->T > 0 ? p->T : 1) * (size_t)p->E;
  const size_t el = elt_size(p);
  w.route = carve_route(c, p, noisy);
  w.blk_cnt = carve_dispatch(c, p);
  const int64_t bm = bwd_gemm_tile_rows(p->dtype);
  w.tile_start = c.take<int32_t>((size_t)p->E + 1 + (size_t)((max_rows_of(p) + bm - 1) / bm + p->E));
  w.topk_idx = c.take<int32_t>(tk);
  w.counts_routed = c.take<int32_t>((size_t)p->E);
  w.counts_kept = c.take<int32_t>((size_t)p->E);
  w.offsets = c.take<int32_t>((size_t)p->E + 1);
  w.slot_dest = c.take<int32_t>(tk);
  w.row_src = c.take<int32_t>(rows);
  w.topk_gate = c.take<float>(tk);
  w.dg = c.take<float>(tk);
  w.dimp = c.take<float>((size_t)p->E);
  w.dload = c.take<float>((size_t)p->E);
  w.dpsw = c.take<float>((size_t)p->E);
  w.dclean = c.take<float>(te);
  w.du = noisy ? c.take<float>(te) : nullptr;
  const int64_t nc = bwd_gate_wgrad_chunks(p->T);
  w.part = c.take<float>((size_t)(nc > 0 ? nc : 1) * (size_t)p->d_model * (size_t)p->E);
  w.part_b = c.take<float>((size_t)(nc > 0 ? nc : 1) * (size_t)p->E);
  w.x_perm = c.take<char>(rows * (size_t)p->d_model * el);
  w.h1 = c.take<char>(rows * (size_t)p->d_ff * el);
  w.d1 = c.take<char>(rows * (size_t)p->d_ff * el);
  w.o = c.take<char>(rows * (size_t)p->d_model * el);
  w.dO = c.take<char>(rows * (size_t)p->d_model * el);
  return w;
}

size_t ws_bytes_for(const moe_params* p, int op, bool noisy) {
  Carver c(nullptr);
  switch (op) {
    case MOE_OP_BACKWARD: carve_backward(c, p, noisy); break;
    case MOE_OP_ROUTE_HIER: carve_route_hier(c, p, true, true); break;
    case MOE_OP_FORWARD_HIER:
      carve_route_hier(c, p, true, true);
      carve_forward(c, p, false);
      break;
    case MOE_OP_ROUTE: carve_route(c, p, noisy); break;
    case MOE_OP_DISPATCH: carve_dispatch(c, p); break;
    case MOE_OP_EXPERT_FFN: carve_ffn(c, p); break;
    default: carve_forward(c, p, noisy); break;
  }
  return (c.off + 255) & ~size_t(255);
}

moe_status check_ws(const moe_params* p, int op, bool noisy, void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(p, op, noisy);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(MOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return MOE_OK;
}

#define REQUIRE_PTR(ptr, name)                                                              \
  do {                                                                                      \
    if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);                       \
    if (!aligned16(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

moe_status check_route_inputs(const moe_params* p, const void* x, const void* w_gate, const void* w_noise,
                              const float* noise) {
  if (p->T > 0) REQUIRE_PTR(x, "x");
  REQUIRE_PTR(w_gate, "w_gate");
  if ((w_noise == nullptr) != (noise == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "w_noise and noise must both be given or both be NULL");
  if (w_noise) {
    REQUIRE_PTR(w_noise, "w_noise");
    if (p->T > 0) REQUIRE_PTR(noise, "noise");
  }
  return MOE_OK;
}

moe_status run_route(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                     const void* w_noise, const float* noise, int32_t* topk_idx, float* topk_gate,
                     int32_t* counts_routed, float* aux_out, float* logits_out, const RouteWs& w, hipStream_t s,
                     bool defer_tail = false) {
  RouteLaunch a;
  a.T = p->T;
  a.d = p->d_model;
  a.E = p->E;
  a.k = p->k;
  a.dtype = p->dtype;
  a.renormalize = p->renormalize;
  a.x = x;
  a.w_gate = w_gate;
  a.gate_bias = gate_bias;
  a.w_noise = w_noise;
  a.noise = noise;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.counts_routed = counts_routed;
  a.aux_out = aux_out;
  a.logits_out = logits_out;
  a.wc = w.wc;
  a.wcat = w.wcat;
  a.gate_mode = p->gate_mode;
  a.lg = w.lg;
  a.part_prob = w.part_prob;
  a.part_imp = w.part_imp;
  a.part_load = w.part_load;
  a.part_cnt = w.part_cnt;
  a.red = w.red;
  a.defer_tail = defer_tail;
  const hipError_t e = launch_route(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "route launch");
}

moe_status run_dispatch(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                        int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm, int32_t* blk_cnt,
                        int32_t* tile_start, bool skip_permute, void* y_zero, hipStream_t s,
                        const RouteWs* route_tail = nullptr, int32_t* counts_routed = nullptr,
                        float* aux_out = nullptr, bool noisy = false) {
  DispatchLaunch a;
  a.T = p->T;
  a.d = p->d_model;
  a.E = p->E;
  a.k = p->k;
  a.dtype = p->dtype;
  a.slot_major = p->drop_order == MOE_DROP_FIRST_CHOICE && p->k > 1 ? 1 : 0;
  a.C = capacity_of(p);
  a.max_rows = max_rows_of(p);
  a.x = x;
  a.topk_idx = topk_idx;
  a.counts_kept = counts_kept;
  a.offsets = offsets;
  a.slot_dest = slot_dest;
  a.row_src = row_src;
  a.x_perm = x_perm;
  a.blk_cnt = blk_cnt;
  a.tile_start = tile_start;
  a.tile_rows = tile_start ? ffn_tile_rows(p->dtype, capacity_of(p), max_rows_of(p), p->E) : 0;
  a.skip_permute = skip_permute;
  a.y_zero = y_zero;
  a.route_tail = route_tail != nullptr;
  a.part_prob = route_tail ? route_tail->part_prob : nullptr;
  a.part_imp = route_tail ? route_tail->part_imp : nullptr;
  a.part_load = route_tail ? route_tail->part_load : nullptr;
  a.part_cnt = route_tail ? route_tail->part_cnt : nullptr;
  a.route_nblk = route_partial_blocks(p->T, p->E, p->dtype, p->gate_mode, false);
  a.counts_routed = counts_routed;
  a.red = route_tail ? route_tail->red : nullptr;
  a.aux_out = aux_out;
  a.noisy = noisy ? 1 : 0;
  const hipError_t e = launch_dispatch(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "dispatch launch");
}

// x_src / row_src (or null): layer 1 gathers its rows from x; y_out / gate (or null,
// top-1 bf16 layers only): layer 2 writes the gated rows straight into y.
moe_status run_ffn(const moe_params* p, const void* x_perm, const int32_t* offsets, const void* w1, const void* w2,
                   void* y_perm, const FfnWs& w, bool tile_map_ready, hipStream_t s, const void* x_src = nullptr,
                   const int32_t* row_src = nullptr, void* y_out = nullptr, const float* gate = nullptr,
                   void* mid_event = nullptr) {
  FfnLaunch a;
  a.d = p->d_model;
  a.f = p->d_ff;
  a.E = p->E;
  a.dtype = p->dtype;
  a.act = p->act;
  a.max_rows = max_rows_of(p);
  a.capacity = capacity_of(p);
  a.x_perm = x_perm;
  a.offsets = offsets;
  a.w1 = w1;
  a.w2 = w2;
  a.y_perm = y_perm;
  a.h1 = w.h1;
  a.tile_start = w.tile_start;
  a.tile_map_ready = tile_map_ready;
  a.x_src = x_src;
  a.row_src = row_src;
  a.T = p->T;
  a.y_out = y_out;
  a.gate = gate;
  a.mid_event = mid_event;
  const hipError_t e = launch_expert_ffn(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert FFN launch");
}

moe_status run_combine(const moe_params* p, const void* y_perm, const int32_t* slot_dest, const float* topk_gate,
                       void* y, hipStream_t s) {
  CombineLaunch a;
  a.T = p->T;
  a.d = p->d_model;
  a.k = p->k;
  a.dtype = p->dtype;
  a.y_perm = y_perm;
  a.slot_dest = slot_dest;
  a.topk_gate = topk_gate;
  a.y = y;
  const hipError_t e = launch_combine(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "combine launch");
}

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
moe_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device ordinal %d >= 64", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t se = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (se != hipSuccess) return hip_fail(se, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return MOE_OK;
}

moe_status check_dispatch_args(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                               int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  REQUIRE_PTR(counts_kept, "counts_kept");
  REQUIRE_PTR(offsets, "offsets");
  if (p->T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(slot_dest, "slot_dest");
    REQUIRE_PTR(row_src, "row_src");
    REQUIRE_PTR(x_perm, "x_perm");
  }
  return MOE_OK;
}

// Everything of the forward after the gate: dispatch (with the route's tail when
// route_tail is given), expert FFN, combine. bf16: the expert GEMM gathers its rows
// from x (no x_perm copy); top-1 layers also write the gated expert outputs
// straight into y (no combine pass; the dispatch zeroes the rows of dropped tokens).
moe_status forward_tail(const moe_params* p, const void* x, const void* w1, const void* w2, void* y, float* aux_out,
                        int32_t* idx, float* gate, int32_t* cr, int32_t* ck, int32_t* sd, const ForwardWs& w,
                        const RouteWs* route_tail, bool noisy, hipStream_t s) {
  moe_status st;
  hipError_t he;
  const bool fused = p->dtype == MOE_BF16;
  const bool direct_y = fused && p->k == 1;
  if ((st = run_dispatch(p, x, idx, ck, w.offsets, sd, w.row_src, w.x_perm, w.blk_cnt, w.ffn.tile_start, fused,
                         direct_y ? y : nullptr, s, route_tail, cr, aux_out, noisy)) != MOE_OK)
    return st;
  if ((he = record_phase(2, s)) != hipSuccess) return hip_fail(he, "phase event");
  if ((st = run_ffn(p, w.x_perm, w.offsets, w1, w2, w.y_perm, w.ffn, true, s, fused ? x : nullptr,
                    fused ? w.row_src : nullptr, direct_y ? y : nullptr, direct_y ? gate : nullptr,
                    g_phase_ev[3])) != MOE_OK)
    return st;
  if ((he = record_phase(4, s)) != hipSuccess) return hip_fail(he, "phase event");
  if (!direct_y && (st = run_combine(p, w.y_perm, sd, gate, y, s)) != MOE_OK) return st;
  if ((he = record_phase(5, s)) != hipSuccess) return hip_fail(he, "phase event");
  return MOE_OK;
}

// The hierarchical gate: both gates' canonical logits, selection, sums, losses.
moe_status run_route_hier(const moe_params* p, const void* x, const void* w_gate_p, const float* gate_bias_p,
                          const void* w_noise_p, const float* noise_p, const void* w_gate_s, const float* gate_bias_s,
                          const void* w_noise_s, const float* noise_s, int32_t* topk_idx, float* topk_gate,
                          int32_t* counts_routed, float* aux_out, const HierWs& w, hipStream_t s) {
  auto logits = [&](int E, const void* wg, const float* b, const void* wn, const float* eps, float* wc, float* lg) {
    RouteLaunch a{};
    a.T = p->T;
    a.d = p->d_model;
    a.E = E;
    a.k = 1;
    a.dtype = p->dtype;
    a.x = x;
    a.w_gate = wg;
    a.gate_bias = b;
    a.w_noise = wn;
    a.noise = eps;
    a.wc = wc;
    a.lg = lg;
    return launch_route_logits(a, s);
  };
  hipError_t he = logits(p->groups, w_gate_p, gate_bias_p, w_noise_p, noise_p, w.wc_p, w.lg_p);
  if (he != hipSuccess) return hip_fail(he, "primary gate launch");
  if ((he = logits(p->E, w_gate_s, gate_bias_s, w_noise_s, noise_s, w.wc_s, w.lg_s)) != hipSuccess)
    return hip_fail(he, "secondary gate launch");
  HierLaunch h{};
  h.T = p->T;
  h.groups = p->groups;
  h.per_group = p->E / p->groups;
  h.k_group = p->k_group;
  h.k_expert = p->k / p->k_group;
  h.noisy_p = w_noise_p != nullptr;
  h.lpad_p = route_logit_pad(p->groups);
  h.lpad_s = route_logit_pad(p->E);
  const size_t np = (size_t)(p->T > 0 ? p->T : 0) * (size_t)h.lpad_p;
  h.Hp = w.lg_p;
  h.CLp = w_noise_p ? w.lg_p + np : nullptr;
  h.SGp = w_noise_p ? w.lg_p + 2 * np : nullptr;
  h.Hs = w.lg_s;
  h.order_p = w.order_p;
  h.gate_p = w.gate_p;
  h.topk_idx = topk_idx;
  h.topk_gate = topk_gate;
  h.counts_routed = counts_routed;
  h.red = w.red;
  h.aux_out = aux_out;
  he = launch_route_hier(h, s);
  return he == hipSuccess ? MOE_OK : hip_fail(he, "hierarchical gate launch");
}

moe_status check_hier_inputs(const moe_params* p, const void* x, const void* w_gate_p, const void* w_noise_p,
                             const float* noise_p, const void* w_gate_s, const void* w_noise_s, const float* noise_s) {
  moe_status st = check_hier(p);
  if (st != MOE_OK) return st;
  if (p->T > 0) REQUIRE_PTR(x, "x");
  REQUIRE_PTR(w_gate_p, "w_gate_p");
  REQUIRE_PTR(w_gate_s, "w_gate_s");
  if ((w_noise_p == nullptr) != (noise_p == nullptr) || (w_noise_s == nullptr) != (noise_s == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "each level's w_noise and noise must both be given or both be NULL");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_capacity(const moe_params* p) {
  if (check_params(p) != MOE_OK) return -2;
  return capacity_of(p);
}

int64_t moe_max_rows(const moe_params* p) {
  if (check_params(p) != MOE_OK) return -1;
  return max_rows_of(p);
}

moe_status moe_workspace_size(const moe_params* p, int op, size_t* bytes) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (op < MOE_OP_ROUTE || op > MOE_OP_FORWARD_HIER) return fail(MOE_ERR_INVALID_ARG, "op = %d", op);
  if ((op == MOE_OP_ROUTE_HIER || op == MOE_OP_FORWARD_HIER) && (st = check_hier(p)) != MOE_OK) return st;
  // The noisy gate uses no extra workspace; size for it either way.
  *bytes = ws_bytes_for(p, op, true);
  return MOE_OK;
}

moe_status moe_route(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                     const void* w_noise, const float* noise, int32_t* topk_idx, float* topk_gate,
                     int32_t* counts_routed, float* aux_out, float* logits_out, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if ((st = check_flat(p)) != MOE_OK) return st;
  if ((st = check_route_inputs(p, x, w_gate, w_noise, noise)) != MOE_OK) return st;
  if (p->T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(topk_gate, "topk_gate");
  }
  REQUIRE_PTR(counts_routed, "counts_routed");
  if (aux_out && !aligned16(aux_out)) return fail(MOE_ERR_INVALID_ARG, "aux_out is not 16-byte aligned");
  if (p->gate_mode == MOE_GATE_EXPORT) {
    if (!logits_out) return fail(MOE_ERR_INVALID_ARG, "MOE_GATE_EXPORT writes into logits_out, which is NULL");
    if (p->dtype != MOE_BF16 || p->E > 256)
      return fail(MOE_ERR_UNSUPPORTED, "MOE_GATE_EXPORT needs the certified MFMA gate (bf16, E <= 256)");
  }
  if ((st = check_ws(p, MOE_OP_ROUTE, w_noise != nullptr, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const RouteWs w = carve_route(c, p, w_noise != nullptr);
  return run_route(p, x, w_gate, gate_bias, w_noise, noise, topk_idx, topk_gate, counts_routed, aux_out,
                   logits_out, w, static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                        int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_dispatch_args(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm);
  if (st != MOE_OK) return st;
  if ((st = check_ws(p, MOE_OP_DISPATCH, false, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  int32_t* blk = carve_dispatch(c, p);
  return run_dispatch(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm, blk, nullptr, false, nullptr,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch_noalloc(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                                int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm, void* stream) {
  moe_status st = check_dispatch_args(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm);
  if (st != MOE_OK) return st;
  const size_t need = ws_bytes_for(p, MOE_OP_DISPATCH, false);
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "the dispatch needs %zu bytes of scratch (E * ceil(T*k/1024) counts), more than the %zu-byte static "
                "scratch of moe_dispatch_noalloc",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MOE_OK) return st;
  // every count the kernels read is written earlier in the same call: nothing to clear
  Carver c(ws);
  int32_t* blk = carve_dispatch(c, p);
  return run_dispatch(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm, blk, nullptr, false, nullptr,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn(const moe_params* p, const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w2, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  REQUIRE_PTR(offsets, "offsets");
  REQUIRE_PTR(w1, "w1");
  REQUIRE_PTR(w2, "w2");
  if (max_rows_of(p) > 0) {
    REQUIRE_PTR(x_perm, "x_perm");
    REQUIRE_PTR(y_perm, "y_perm");
  }
  if ((st = check_ws(p, MOE_OP_EXPERT_FFN, false, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const FfnWs w = carve_ffn(c, p);
  return run_ffn(p, x_perm, offsets, w1, w2, y_perm, w, false, static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_params* p, const void* y_perm, const int32_t* slot_dest, const float* topk_gate,
                       void* y, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if (p->T > 0) {
    REQUIRE_PTR(slot_dest, "slot_dest");
    REQUIRE_PTR(topk_gate, "topk_gate");
    REQUIRE_PTR(y, "y");
    if (max_rows_of(p) > 0) REQUIRE_PTR(y_perm, "y_perm");
  }
  return run_combine(p, y_perm, slot_dest, topk_gate, y, static_cast<hipStream_t>(stream));
}

moe_status moe_forward(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                       const void* w_noise, const float* noise, const void* w1, const void* w2, void* y,
                       float* aux_out, int32_t* topk_idx, float* topk_gate, int32_t* counts_routed,
                       int32_t* counts_kept, int32_t* slot_dest, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if ((st = check_flat(p)) != MOE_OK) return st;
  if ((st = check_route_inputs(p, x, w_gate, w_noise, noise)) != MOE_OK) return st;
  REQUIRE_PTR(w1, "w1");
  REQUIRE_PTR(w2, "w2");
  if (p->T > 0) REQUIRE_PTR(y, "y");
  const void* opt[] = {aux_out, topk_idx, topk_gate, counts_routed, counts_kept, slot_dest};
  for (const void* q : opt)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "an optional output is not 16-byte aligned");
  const bool noisy = w_noise != nullptr;
  if ((st = check_ws(p, MOE_OP_FORWARD, noisy, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const ForwardWs w = carve_forward(c, p, noisy);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : w.topk_idx;
  float* gate = topk_gate ? topk_gate : w.topk_gate;
  int32_t* cr = counts_routed ? counts_routed : w.counts_routed;
  int32_t* ck = counts_kept ? counts_kept : w.counts_kept;
  int32_t* sd = slot_dest ? slot_dest : w.slot_dest;
  hipError_t he;
  if ((he = record_phase(0, s)) != hipSuccess) return hip_fail(he, "phase event");
  // the route's per-expert sums and losses run inside the dispatch kernels
  if ((st = run_route(p, x, w_gate, gate_bias, w_noise, noise, idx, gate, cr, aux_out, nullptr, w.route, s, true)) !=
      MOE_OK)
    return st;
  if ((he = record_phase(1, s)) != hipSuccess) return hip_fail(he, "phase event");
  return forward_tail(p, x, w1, w2, y, aux_out, idx, gate, cr, ck, sd, w, &w.route, noisy, s);
}

moe_status moe_backward(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                        const void* w_noise, const float* noise, const void* w1, const void* w2, const void* dy,
                        double w_switch, double w_importance, double w_load, void* dx, float* dw_gate,
                        float* dgate_bias, float* dw_noise, void* dw1, void* dw2, float* dlogits, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if ((st = check_flat(p)) != MOE_OK) return st;
  if ((st = check_route_inputs(p, x, w_gate, w_noise, noise)) != MOE_OK) return st;
  REQUIRE_PTR(w1, "w1");
  REQUIRE_PTR(w2, "w2");
  REQUIRE_PTR(dw_gate, "dw_gate");
  REQUIRE_PTR(dw1, "dw1");
  REQUIRE_PTR(dw2, "dw2");
  if (p->T > 0) {
    REQUIRE_PTR(dy, "dy");
    REQUIRE_PTR(dx, "dx");
  }
  const bool noisy = w_noise != nullptr;
  if (noisy) REQUIRE_PTR(dw_noise, "dw_noise");
  if (dgate_bias && !aligned16(dgate_bias)) return fail(MOE_ERR_INVALID_ARG, "dgate_bias is not 16-byte aligned");
  if (dlogits && !aligned16(dlogits)) return fail(MOE_ERR_INVALID_ARG, "dlogits is not 16-byte aligned");
  if (!(isfinite(w_switch) && isfinite(w_importance) && isfinite(w_load)))
    return fail(MOE_ERR_INVALID_ARG, "loss weights must be finite");
  if ((st = check_ws(p, MOE_OP_BACKWARD, noisy, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const BackwardWs w = carve_backward(c, p, noisy);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the gate on its canonical fp32 path, which keeps H, the clean logits and the
  // softplus values; the same routing as the forward in every gate mode
  moe_params pc = *p;
  pc.gate_mode = MOE_GATE_CANONICAL;
  if ((st = run_route(&pc, x, w_gate, gate_bias, w_noise, noise, w.topk_idx, w.topk_gate, w.counts_routed, nullptr,
                      nullptr, w.route, s)) != MOE_OK)
    return st;
  if ((st = run_dispatch(p, x, w.topk_idx, w.counts_kept, w.offsets, w.slot_dest, w.row_src, w.x_perm, w.blk_cnt,
                         nullptr, false, nullptr, s)) != MOE_OK)
    return st;
  const int bm = bwd_gemm_tile_rows(p->dtype), bn = bwd_gemm_tile_cols(p->dtype);
  hipError_t he = launch_tile_map(w.offsets, p->E, bm, w.tile_start, s);
  if (he != hipSuccess) return hip_fail(he, "tile map launch");
  const int64_t R = max_rows_of(p);
  const int d = p->d_model, f = p->d_ff;
  const uint32_t el = (uint32_t)elt_size(p);
  const int64_t mtiles = (R + bm - 1) / bm + p->E;
  auto seg_m = [&](const void* A, int64_t lda, const void* B, int64_t ldb, void* C, void* C2, const void* Dm,
                   int N, int K) {
    BwdGemmArgs g{};
    g.A = static_cast<const uint16_t*>(A);
    g.B = static_cast<const uint16_t*>(B);
    g.C = static_cast<uint16_t*>(C);
    g.C2 = static_cast<uint16_t*>(C2);
    g.Dmul = static_cast<const uint16_t*>(Dm);
    g.offsets = w.offsets;
    g.tile_start = w.tile_start;
    g.E = p->E;
    g.N = N;
    g.K = K;
    g.n_tiles_n = (N + bn - 1) / bn;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = N;
    g.b_expert_stride = (int64_t)d * f;
    g.a_bytes = (uint32_t)(R * lda * el);
    return g;
  };
  auto run = [&](BwdGemmKind kind, const BwdGemmArgs& g, int64_t blocks, const char* what) -> moe_status {
    const hipError_t e = launch_bwd_gemm(kind, g, blocks, p->dtype, p->act, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, what);
  };
  // recompute the expert FFN: H1 = act(Xp W1), D1 = act'(Xp W1), O = H1 W2
  BwdGemmArgs g = seg_m(w.x_perm, d, w1, f, w.h1, w.d1, nullptr, f, d);
  if ((st = run(kBwdRecompute1, g, mtiles * g.n_tiles_n, "expert backward launch")) != MOE_OK) return st;
  g = seg_m(w.h1, f, w2, d, w.o, nullptr, nullptr, d, f);
  if ((st = run(kBwdRecompute2, g, mtiles * g.n_tiles_n, "expert backward launch")) != MOE_OK) return st;
  // combine adjoint (dO = g dy), dL/dg, and the gate's backward
  BwdMiscArgs b{};
  b.T = p->T;
  b.d = d;
  b.E = p->E;
  b.k = p->k;
  b.dtype = p->dtype;
  b.renormalize = p->renormalize;
  b.noisy = noisy ? 1 : 0;
  b.lpad = (p->E + 3) & ~3;
  b.x = x;
  b.w_gate = w_gate;
  b.w_noise = w_noise;
  b.noise = noise;
  b.dy = dy;
  b.o = w.o;
  b.dO = w.dO;
  b.slot_dest = w.slot_dest;
  b.topk_idx = w.topk_idx;
  b.topk_gate = w.topk_gate;
  b.dg = w.dg;
  b.red = w.route.red;
  b.counts_routed = w.counts_routed;
  b.w_switch = w_switch;
  b.w_imp = w_importance;
  b.w_load = w_load;
  b.dimp = w.dimp;
  b.dload = w.dload;
  b.dpsw = w.dpsw;
  const size_t lpn = (size_t)(p->T > 0 ? p->T : 0) * (size_t)b.lpad;
  b.H = w.route.lg;
  b.CL = noisy ? w.route.lg + lpn : nullptr;
  b.SG = noisy ? w.route.lg + 2 * lpn : nullptr;
  b.dclean = dlogits ? dlogits : w.dclean;
  b.du = w.du;
  b.dxp = w.o;
  b.dx = dx;
  if ((he = launch_bwd_gather(b, s)) != hipSuccess) return hip_fail(he, "backward gather launch");
  if ((he = launch_bwd_gate(b, s)) != hipSuccess) return hip_fail(he, "gate backward launch");
  // data gradients: dZ = (dO W2^T) * act'(z) (in place over D1), dXp = dZ W1^T (over O)
  g = seg_m(w.dO, d, w2, d, w.d1, nullptr, w.d1, f, d);
  if ((st = run(kBwdDataGrad2, g, mtiles * g.n_tiles_n, "expert backward launch")) != MOE_OK) return st;
  g = seg_m(w.d1, f, w1, f, w.o, nullptr, nullptr, d, f);
  if ((st = run(kBwdDataGrad1, g, mtiles * g.n_tiles_n, "expert backward launch")) != MOE_OK) return st;
  // weight gradients over each expert's rows: dW2 = H1^T dO, dW1 = Xp^T dZ
  auto seg_k = [&](const void* A, int M, const void* B, int N, void* C) {
    BwdGemmArgs q{};
    q.A = static_cast<const uint16_t*>(A);
    q.B = static_cast<const uint16_t*>(B);
    q.C = static_cast<uint16_t*>(C);
    q.offsets = w.offsets;
    q.E = p->E;
    q.M = M;
    q.N = N;
    q.n_tiles_m = (M + bm - 1) / bm;
    q.n_tiles_n = (N + bn - 1) / bn;
    q.lda = M;
    q.ldb = N;
    q.ldc = N;
    q.c_expert_stride = (int64_t)M * N;
    q.a_bytes = (uint32_t)(R * M * el);
    q.b_bytes = (uint32_t)(R * N * el);
    return q;
  };
  g = seg_k(w.h1, f, w.dO, d, dw2);
  if ((st = run(kBwdWeightGrad, g, (int64_t)p->E * g.n_tiles_m * g.n_tiles_n, "weight gradient launch")) != MOE_OK)
    return st;
  g = seg_k(w.x_perm, d, w.d1, f, dw1);
  if ((st = run(kBwdWeightGrad, g, (int64_t)p->E * g.n_tiles_m * g.n_tiles_n, "weight gradient launch")) != MOE_OK)
    return st;
  // gate weight gradients and dx
  if ((he = launch_bwd_gate_wgrad(b, b.dclean, dw_gate, gate_bias ? dgate_bias : nullptr, w.part, w.part_b, s)) !=
      hipSuccess)
    return hip_fail(he, "gate weight gradient launch");
  if (noisy && (he = launch_bwd_gate_wgrad(b, w.du, dw_noise, nullptr, w.part, w.part_b, s)) != hipSuccess)
    return hip_fail(he, "noise weight gradient launch");
  if ((he = launch_bwd_dx(b, s)) != hipSuccess) return hip_fail(he, "dx launch");
  return MOE_OK;
}

moe_status moe_route_hier(const moe_params* p, const void* x, const void* w_gate_p, const float* gate_bias_p,
                          const void* w_noise_p, const float* noise_p, const void* w_gate_s, const float* gate_bias_s,
                          const void* w_noise_s, const float* noise_s, int32_t* topk_idx, float* topk_gate,
                          int32_t* counts_routed, float* aux_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if ((st = check_hier_inputs(p, x, w_gate_p, w_noise_p, noise_p, w_gate_s, w_noise_s, noise_s)) != MOE_OK) return st;
  if (p->T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(topk_gate, "topk_gate");
  }
  REQUIRE_PTR(counts_routed, "counts_routed");
  if (aux_out && !aligned16(aux_out)) return fail(MOE_ERR_INVALID_ARG, "aux_out is not 16-byte aligned");
  if ((st = check_ws(p, MOE_OP_ROUTE_HIER, true, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const HierWs w = carve_route_hier(c, p, true, true);
  return run_route_hier(p, x, w_gate_p, gate_bias_p, w_noise_p, noise_p, w_gate_s, gate_bias_s, w_noise_s, noise_s,
                        topk_idx, topk_gate, counts_routed, aux_out, w, static_cast<hipStream_t>(stream));
}

moe_status moe_forward_hier(const moe_params* p, const void* x, const void* w_gate_p, const float* gate_bias_p,
                            const void* w_noise_p, const float* noise_p, const void* w_gate_s,
                            const float* gate_bias_s, const void* w_noise_s, const float* noise_s, const void* w1,
                            const void* w2, void* y, float* aux_out, int32_t* topk_idx, float* topk_gate,
                            int32_t* counts_routed, int32_t* counts_kept, int32_t* slot_dest, void* ws,
                            size_t ws_bytes, void* stream) {
  moe_status st = check_params(p);
  if (st != MOE_OK) return st;
  if ((st = check_hier_inputs(p, x, w_gate_p, w_noise_p, noise_p, w_gate_s, w_noise_s, noise_s)) != MOE_OK) return st;
  REQUIRE_PTR(w1, "w1");
  REQUIRE_PTR(w2, "w2");
  if (p->T > 0) REQUIRE_PTR(y, "y");
  const void* opt[] = {aux_out, topk_idx, topk_gate, counts_routed, counts_kept, slot_dest};
  for (const void* q : opt)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "an optional output is not 16-byte aligned");
  if ((st = check_ws(p, MOE_OP_FORWARD_HIER, true, ws, ws_bytes)) != MOE_OK) return st;
  Carver c(ws);
  const HierWs wr = carve_route_hier(c, p, true, true);
  const ForwardWs w = carve_forward(c, p, false);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : w.topk_idx;
  float* gate = topk_gate ? topk_gate : w.topk_gate;
  int32_t* cr = counts_routed ? counts_routed : w.counts_routed;
  int32_t* ck = counts_kept ? counts_kept : w.counts_kept;
  int32_t* sd = slot_dest ? slot_dest : w.slot_dest;
  hipError_t he;
  if ((he = record_phase(0, s)) != hipSuccess) return hip_fail(he, "phase event");
  if ((st = run_route_hier(p, x, w_gate_p, gate_bias_p, w_noise_p, noise_p, w_gate_s, gate_bias_s, w_noise_s, noise_s,
                           idx, gate, cr, aux_out, wr, s)) != MOE_OK)
    return st;
  if ((he = record_phase(1, s)) != hipSuccess) return hip_fail(he, "phase event");
  return forward_tail(p, x, w1, w2, y, nullptr, idx, gate, cr, ck, sd, w, nullptr, false, s);
}

// Phase events of moe_forward on the calling thread (n = 0 or events NULL: off).
moe_status moe_set_phase_events(void* const* events, int n) {
  if (n < 0 || n > kPhaseEvents) return fail(MOE_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, kPhaseEvents);
  for (int i = 0; i < kPhaseEvents; ++i) g_phase_ev[i] = (events && i < n) ? events[i] : nullptr;
  return MOE_OK;
}

// Counter-based standard-normal noise (see include/moe.h).
moe_status moe_standard_normal(uint64_t seed, int64_t row0, int64_t rows, int32_t cols, float* out, void* stream) {
  if (rows < 0 || cols < 0 || row0 < 0) return fail(MOE_ERR_INVALID_ARG, "rows, cols and row0 must be >= 0");
  if (rows * (int64_t)cols > 0 && !out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  if (rows > 0 && (uint64_t)(row0 + rows - 1) < (uint64_t)row0) return fail(MOE_ERR_INVALID_ARG, "row range overflows");
  const hipError_t e = launch_normal_noise(seed, row0, rows, cols, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "noise launch");
}

// Canonical softplus of the noisy gate, element-wise (z, out: n fp32 device values).
moe_status moe_canonical_softplus(const float* z, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n > 0 && (!z || !out)) return fail(MOE_ERR_INVALID_ARG, "z or out is NULL");
  const hipError_t e = launch_softplus(z, out, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "softplus launch");
}

}  // extern "C"
