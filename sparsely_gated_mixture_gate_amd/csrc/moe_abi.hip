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
  if (p->gate_mode < MOE_GATE_AUTO || p->gate_mode > MOE_GATE_FALLBACK)
    return fail(MOE_ERR_INVALID_ARG, "gate_mode = %d (0, 1 or 2)", p->gate_mode);
  if (p->T * (int64_t)p->k >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld >= 2^31", (long long)(p->T * p->k));
  if (isnan(p->capacity_factor)) return fail(MOE_ERR_INVALID_ARG, "capacity_factor is NaN");
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

size_t ws_bytes_for(const moe_params* p, int op, bool noisy) {
  Carver c(nullptr);
  switch (op) {
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
  if (op < MOE_OP_ROUTE || op > MOE_OP_FORWARD) return fail(MOE_ERR_INVALID_ARG, "op = %d", op);
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
  if ((st = check_route_inputs(p, x, w_gate, w_noise, noise)) != MOE_OK) return st;
  if (p->T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(topk_gate, "topk_gate");
  }
  REQUIRE_PTR(counts_routed, "counts_routed");
  if (aux_out && !aligned16(aux_out)) return fail(MOE_ERR_INVALID_ARG, "aux_out is not 16-byte aligned");
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
  // bf16: the expert GEMM gathers its rows from x (no x_perm copy); top-1 layers also
  // write the gated expert outputs straight into y (no combine pass; the dispatch
  // zeroes the rows of dropped tokens)
  const bool fused = p->dtype == MOE_BF16;
  const bool direct_y = fused && p->k == 1;
  if ((st = run_dispatch(p, x, idx, ck, w.offsets, sd, w.row_src, w.x_perm, w.blk_cnt, w.ffn.tile_start, fused,
                         direct_y ? y : nullptr, s, &w.route, cr, aux_out, noisy)) != MOE_OK)
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

// Phase events of moe_forward on the calling thread (n = 0 or events NULL: off).
moe_status moe_set_phase_events(void* const* events, int n) {
  if (n < 0 || n > kPhaseEvents) return fail(MOE_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, kPhaseEvents);
  for (int i = 0; i < kPhaseEvents; ++i) g_phase_ev[i] = (events && i < n) ? events[i] : nullptr;
  return MOE_OK;
}

// Canonical softplus of the noisy gate, element-wise (z, out: n fp32 device values).
moe_status moe_canonical_softplus(const float* z, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n > 0 && (!z || !out)) return fail(MOE_ERR_INVALID_ARG, "z or out is NULL");
  const hipError_t e = launch_softplus(z, out, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "softplus launch");
}

}  // extern "C"
