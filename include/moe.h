/*
 * moe.h -- C ABI of the gfx950 (MI355X) forward pass of one sparsely-gated
 * Mixture-of-Experts layer.
 *
 * The layer, from the pages:
 *   - Shazeer et al. summary page ("Outrageously Large Neural Networks: The
 *     Sparsely-Gated Mixture-of-Experts Layer"), section "Methode": the layer
 *     output y = sum_i G(x)_i E_i(x), skipping experts whose gate is zero;
 *     noisy top-k gating H(x)_i = (x W_g)_i + StandardNormal() *
 *     Softplus((x W_noise)_i), G(x) = Softmax(KeepTopK(H(x), k)); and the
 *     importance / load balancing losses, CV(.)^2 of per-expert sums.
 *   - "Switch Transformer" page: top-1 routing; its listing takes the softmax
 *     over all experts, keeps the top-1 probability as the gate and gathers
 *     each expert's tokens; an auxiliary load-balancing loss is named.
 *   - "moe paper models" page, table 2: capacity factors (1.25, 1/1.5/2x, 2).
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer to contiguous row-major data,
 *     aligned to 16 bytes, owned by the caller, unless stated otherwise. The
 *     library allocates no device memory and keeps no state between calls
 *     except a thread-local error string and the thread-local phase events of
 *     moe_set_phase_events.
 *   - "dtype" tensors (x, w_gate, w_noise, w1, w2, x_perm, y_perm, y) are all
 *     bf16 (raw 16-bit patterns) or all fp32, per moe_params.dtype. Logits,
 *     gates, noise, gate_bias and aux are always fp32; indices are int32.
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronising. Outputs are valid once the
 *     stream reaches them.
 *   - Errors: arguments are checked before anything is enqueued; a failing
 *     check returns MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED or
 *     MOE_ERR_WORKSPACE, enqueues nothing, and sets moe_last_error(). A failed
 *     launch returns MOE_ERR_HIP. Faults inside kernels surface at the
 *     caller's next synchronisation. Capacity overflow is not an error: the
 *     overflowing assignments are dropped.
 *   - Preconditions not checked on the device: inputs finite (no NaN/Inf);
 *     pointers valid for the documented extents.
 *   - Supported domain: T >= 0, T*k < 2^31, 1 <= E <= 1024, 1 <= k <= min(E, 8),
 *     d_model and d_ff positive multiples of 8.
 *   - Workspace: `ws` is caller-owned device scratch of at least
 *     moe_workspace_size() bytes for that entry point, 256-byte aligned. Two
 *     calls that may run at the same time need separate workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a pointer, size or option outside the documented domain */
  MOE_ERR_UNSUPPORTED = 2, /* outside the supported domain (e.g. d_model % 8 != 0, E > 1024) */
  MOE_ERR_WORKSPACE = 3,   /* ws NULL, misaligned or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status;

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ACT_RELU = 0, MOE_ACT_GELU = 1 }; /* GELU is the exact 0.5 z (1 + erf(z / sqrt 2)) */
enum {
  MOE_OP_ROUTE = 0, MOE_OP_DISPATCH = 1, MOE_OP_EXPERT_FFN = 2, MOE_OP_FORWARD = 3, MOE_OP_BACKWARD = 4,
  MOE_OP_ROUTE_HIER = 5, MOE_OP_FORWARD_HIER = 6
};
enum { MOE_GATE_AUTO = 0, MOE_GATE_CANONICAL = 1, MOE_GATE_FALLBACK = 2, MOE_GATE_EXPORT = 3 };
enum { MOE_DROP_TOKEN_ORDER = 0, MOE_DROP_FIRST_CHOICE = 1 };

typedef struct moe_params {
  int64_t T;               /* tokens in the batch */
  int32_t d_model;         /* token width d */
  int32_t d_ff;            /* expert hidden width f */
  int32_t E;               /* number of experts */
  int32_t k;               /* experts per token */
  int32_t dtype;           /* MOE_F32 or MOE_BF16 */
  int32_t act;             /* MOE_ACT_RELU or MOE_ACT_GELU */
  int32_t renormalize;     /* 1: gates = softmax over the k kept logits (Shazeer, KeepTopK + Softmax);
                              0: gates = full-softmax probabilities of the kept experts (Switch listing) */
  int32_t gate_mode;       /* how moe_route / moe_forward evaluate the gate logits (MOE_GATE_*):
                              MOE_GATE_AUTO (0): bf16 layers with E <= 256 compute the logits with
                                bf16 MFMAs and certify each token's top-k against the canonical
                                logits (below); uncertified tokens, fp32 layers, E > 256 and calls
                                with logits_out use the canonical fp32 chains;
                              MOE_GATE_CANONICAL (1): canonical fp32 chains for every token;
                              MOE_GATE_FALLBACK (2): the MFMA path with every token sent through its
                                canonical fallback (testing);
                              MOE_GATE_EXPORT (3, moe_route only; bf16, E <= 256): MOE_GATE_AUTO,
                                and logits_out [2][T][E] receives the certificate's inputs: the MFMA
                                logits H (before any recompute) and, per entry, the bound on their
                                distance to the canonical logits (auditing). Routing is identical in
                                all modes. */
  double capacity_factor;  /* > 0: per-expert capacity C = ceil(capacity_factor * k * T / E); <= 0: none */
  int64_t capacity;        /* >= 0: explicit per-expert capacity C (overrides capacity_factor); < 0: unused */
  int32_t drop_order;      /* which assignments a full expert drops (MOE_DROP_*):
                              MOE_DROP_TOKEN_ORDER (0): tokens in order, slots in order within a token;
                                the first C assignments of an expert are kept;
                              MOE_DROP_FIRST_CHOICE (1): first-choice priority ("moe paper models"
                                table 2, GShard row: top-2 with a capacity): slot 0 of every token in
                                token order, then slot 1 of every token, ...; ranks and the rows of
                                each expert's segment follow that order. Same as 0 when k = 1. */
  int32_t groups;          /* hierarchical layers (moe_route_hier / moe_forward_hier): the number of
                              secondary MoE groups g >= 1, each of E / g experts; 0 or 1 for a flat
                              layer (the flat gate's entry points reject groups > 1) */
  int32_t k_group;         /* hierarchical layers: groups the primary gate keeps (k_group <= groups);
                              each kept group keeps k / k_group of its experts, so k is the total
                              number of expert slots of a token */
} moe_params;

/* Human-readable name of a status code. Never NULL; static storage. */
const char* moe_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Per-expert capacity C for p (see moe_params), -1 if unlimited, -2 if p is
 * invalid. Host-only; no HIP call. */
int64_t moe_capacity(const moe_params* p);

/* Upper bound on kept rows R = sum_e min(routed_e, C): min(T*k, E*C). Sizes
 * x_perm / y_perm / row_src. Host-only. Returns -1 if p is invalid. */
int64_t moe_max_rows(const moe_params* p);

/* Workspace bytes needed by entry point `op` (MOE_OP_*) for p. Host-only. */
moe_status moe_workspace_size(const moe_params* p, int op, size_t* bytes);

/*
 * moe_route -- gate logits, top-k, gate values, routed counts, balancing losses.
 *   (Shazeer "Methode": Noisy Top-K Gating and Load-Balancing-Losses;
 *    Switch page: softmax over all experts and top-1.)
 * Logits, in fp32 with a fixed order of operations (the order is part of the
 * contract; it makes the integer routing reproducible bit-for-bit):
 *   clean[t,e] = (sum_{j=0..d-1, ascending} fma-accumulated x[t,j]*w_gate[j,e]) (+ gate_bias[e])
 *   H[t,e]     = fma(noise[t,e], softplus(x[t,:] . w_noise[:,e]), clean[t,e])   if w_noise
 *              = clean[t,e]                                                    otherwise
 * with the dot products accumulated from +0 in ascending j, one fma per term,
 * and softplus built from IEEE fp32 basic operations (exp by Cody-Waite
 * reduction + degree-7 Taylor/Horner, log1p via 2*atanh(v/(2+v)) with a
 * degree-8 odd series; z > 20 returns z; exp is 0 below -87).
 * Experts are ordered by H descending, ties to the lower index; slot s < k
 * takes the s-th. Gates (fp32): renormalize=1: softmax over the kept logits;
 * 0: full-softmax probability.
 * Certified MFMA gate (gate_mode AUTO, bf16, E <= 256, logits_out NULL): the
 * logits are computed with bf16 MFMAs (exact products, fp32 sums in the
 * hardware's order) together with S = sum_j |x[t,j] w[j,e]| and Q = the sum of
 * |accumulator| over the M = ceil(d/32) k-steps, which bound the distance to the
 * canonical value by B = 100 2^-24 (Q + S)(1 + 256 2^-24 M) (plus the rounding of
 * the bias add, softplus and fma). A token whose k gaps between consecutive
 * values of its top-(k+1) all exceed twice its largest B has the canonical
 * routing. For every other token, the experts whose MFMA value lies within 2B
 * of its (k+1)-th value (the only ones that can be in the canonical top-(k+1))
 * get their logits recomputed with the canonical chains, or the whole row is
 * recomputed where those do not fit, and the token is selected again. topk_idx
 * and counts_routed are therefore those of the canonical logits in every mode;
 * the gates, aux losses and load estimates use the MFMA logits where they were
 * not recomputed (rounding-level differences).
 * Inputs:  x [T,d] dtype; w_gate [d,E] dtype; gate_bias [E] fp32 or NULL;
 *          w_noise [d,E] dtype or NULL; noise [T,E] fp32 standard normals
 *          (required iff w_noise).
 * Outputs: topk_idx [T,k] int32; topk_gate [T,k] fp32;
 *          counts_routed [E] int32 (assignments per expert, before capacity);
 *          aux_out [3] fp32 or NULL: {E*sum_e f_e*P_e with f_e = routed_e/(T*k) and
 *            P_e = mean_t softmax(H_t)_e; CV^2 of importance_e = sum of the gates
 *            routed to e; CV^2 of load_e = sum_t Phi((clean[t,e] - kth_excluding(H_t,k,e))
 *            / softplus(...)) -- NaN without w_noise}; CV^2 uses the population variance;
 *          logits_out [T,E] fp32 (H) or NULL.
 */
moe_status moe_route(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                     const void* w_noise, const float* noise, int32_t* topk_idx, float* topk_gate,
                     int32_t* counts_routed, float* aux_out, float* logits_out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_dispatch -- group assignments by expert with capacity drops in token order.
 *   (Switch listing: per-expert gather of the routed tokens; "moe paper
 *    models" table 2: capacity factors.)
 * The T*k assignments are walked in token order (slot order within a token),
 * or slot-major with drop_order = MOE_DROP_FIRST_CHOICE; each takes the next
 * rank of its expert; rank >= C is dropped.
 * Inputs:  x [T,d] dtype; topk_idx [T,k] int32 (values in [0,E), distinct per token).
 * Outputs: counts_kept [E] int32 = min(routed_e, C);
 *          offsets [E+1] int32, exclusive prefix sum of counts_kept (offsets[E] = R);
 *          slot_dest [T,k] int32: row of the assignment in x_perm, or -1 if dropped;
 *          row_src [moe_max_rows] int32: token of each row (entries >= R untouched);
 *          x_perm [moe_max_rows, d] dtype: x_perm[r] = x[row_src[r]] (rows >= R untouched).
 * Rows are sorted by (expert, token), or (expert, slot, token) with first-choice priority.
 */
moe_status moe_dispatch(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                        int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch with no workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same inputs, outputs,
 * layouts and results as moe_dispatch.
 * Its scratch (the per-block expert counts) lives in a fixed 1 MiB device array
 * inside the library, one copy per GPU, held until the process ends; the first
 * call on a device looks up that device's copy. The call allocates nothing.
 * Limit: E * ceil(T*k / 1024) * 4 bytes (rounded up to 256) <= 1 MiB, else
 * MOE_ERR_UNSUPPORTED before anything is enqueued (e.g. E = 256 allows
 * T*k <= 1,048,576). Every call on a GPU shares that GPU's array: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller. Nothing in the array needs to start at zero.
 */
moe_status moe_dispatch_noalloc(const moe_params* p, const void* x, const int32_t* topk_idx, int32_t* counts_kept,
                                int32_t* offsets, int32_t* slot_dest, int32_t* row_src, void* x_perm, void* stream);

/*
 * moe_expert_ffn -- every expert's two-layer FFN on its contiguous row segment.
 *   (Shazeer abstract / "Methode": experts are feed-forward sub-networks.)
 *   y_perm[r] = act(x_perm[r] . w1[e]) . w2[e] for offsets[e] <= r < offsets[e+1],
 * no biases; products accumulate in fp32; for bf16 the hidden activation is
 * rounded to bf16 (nearest-even) before the second product.
 * Inputs:  x_perm [R,d] dtype; offsets [E+1] int32 (device; R = offsets[E] <= moe_max_rows);
 *          w1 [E,d,f] dtype; w2 [E,f,d] dtype.
 * Outputs: y_perm [R,d] dtype (rows >= R untouched).
 */
moe_status moe_expert_ffn(const moe_params* p, const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w2, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- gate-weighted sum back into token order.
 *   (Shazeer "Methode": y = sum_i G(x)_i E_i(x); Switch listing: expert outputs
 *    added back at their tokens.)
 *   y[t] = sum over s = 0..k-1 with slot_dest[t,s] >= 0 of topk_gate[t,s] * y_perm[slot_dest[t,s]],
 * accumulated in fp32 in slot order; a token with every slot dropped gets 0.
 * Dropped gates are not redistributed.
 * Inputs:  y_perm [R,d] dtype; slot_dest [T,k] int32; topk_gate [T,k] fp32.
 * Outputs: y [T,d] dtype.
 */
moe_status moe_combine(const moe_params* p, const void* y_perm, const int32_t* slot_dest, const float* topk_gate,
                       void* y, void* stream);

/*
 * moe_forward -- the whole layer: moe_route, moe_dispatch, moe_expert_ffn and
 * moe_combine on one stream, intermediates in `ws`. For bf16 layers the expert
 * GEMM reads its rows straight from x (x_perm is not materialised); for top-1
 * bf16 layers it also writes y[t] = topk_gate[t] * (expert output) directly, in
 * fp32 rounded once to bf16 (moe_combine would round the expert output to bf16
 * first), and the rows of dropped tokens are zeroed by the dispatch.
 * Inputs as moe_route plus w1, w2. Outputs: y [T,d] dtype (required);
 * aux_out [3], topk_idx [T,k], topk_gate [T,k], counts_routed [E], counts_kept [E],
 * slot_dest [T,k] -- each optional (NULL: kept in the workspace only).
 */
moe_status moe_forward(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                       const void* w_noise, const float* noise, const void* w1, const void* w2, void* y,
                       float* aux_out, int32_t* topk_idx, float* topk_gate, int32_t* counts_routed,
                       int32_t* counts_kept, int32_t* slot_dest, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_hier -- the gate of a hierarchical MoE layer.
 *   (Shazeer summary page, "Schluesselbegriffe": a primary gating network routes
 *    each input to secondary MoE groups; "moe paper models" table 2: k = 2 for
 *    the hierarchical models.)
 * The layer is a MoE of MoEs, y = sum_i Gp(x)_i sum_j G_i(x)_j E_ij(x), with both
 * gates noisy top-k gates of the "Methode" section (softmax over the kept logits):
 *   primary:   Hp = x w_gate_p (+ gate_bias_p) (+ noise_p * softplus(x w_noise_p)),
 *              over p->groups groups, keeps p->k_group of them;
 *   secondary: Hs = x w_gate_s (+ gate_bias_s) (+ noise_s * softplus(x w_noise_s)),
 *              over all E experts (column g * b + j is expert j of group g,
 *              b = E / groups); each kept group keeps its top k / k_group.
 * Logits are the canonical fp32 chains of moe_route; top-k ties go to the lower
 * index. Slot r * (k / k_group) + q of a token is expert q of its r-th kept group:
 * topk_idx = g * b + j, topk_gate = Gp_g * G_g,j. moe_dispatch, moe_expert_ffn
 * and moe_combine then treat the layer as a flat one with E experts and k slots.
 * Inputs:  x [T,d] dtype; w_gate_p [d,groups], w_gate_s [d,E] dtype; gate_bias_p
 *          [groups], gate_bias_s [E] fp32 or NULL; w_noise_p [d,groups] + noise_p
 *          [T,groups] and w_noise_s [d,E] + noise_s [T,E] (fp32 standard normals),
 *          each pair both or neither.
 * Outputs: topk_idx, topk_gate [T,k]; counts_routed [E]; aux_out [3] or NULL:
 *          {CV^2 of the primary importance (per group), CV^2 of the importance of
 *          the combined gates (per expert), CV^2 of the primary load estimate
 *          (NaN without w_noise_p)} (population CV, unweighted).
 * Requires groups >= 1 dividing E, k_group >= 1 dividing k, k_group <= groups,
 * k / k_group <= E / groups. renormalize and gate_mode are not used.
 * Workspace: moe_workspace_size(p, MOE_OP_ROUTE_HIER).
 */
moe_status moe_route_hier(const moe_params* p, const void* x, const void* w_gate_p, const float* gate_bias_p,
                          const void* w_noise_p, const float* noise_p, const void* w_gate_s, const float* gate_bias_s,
                          const void* w_noise_s, const float* noise_s, int32_t* topk_idx, float* topk_gate,
                          int32_t* counts_routed, float* aux_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_hier -- the whole hierarchical layer: moe_route_hier, then the
 * dispatch, expert FFN and combine of moe_forward (E experts, k slots).
 * Inputs as moe_route_hier plus w1 [E,d,f], w2 [E,f,d]; outputs as moe_forward
 * (aux_out as moe_route_hier). Workspace: moe_workspace_size(p, MOE_OP_FORWARD_HIER).
 */
moe_status moe_forward_hier(const moe_params* p, const void* x, const void* w_gate_p, const float* gate_bias_p,
                            const void* w_noise_p, const float* noise_p, const void* w_gate_s,
                            const float* gate_bias_s, const void* w_noise_s, const float* noise_s, const void* w1,
                            const void* w2, void* y, float* aux_out, int32_t* topk_idx, float* topk_gate,
                            int32_t* counts_routed, int32_t* counts_kept, int32_t* slot_dest, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * moe_backward -- gradients of the layer (the pages train it: Shazeer
 *   "Fragen" -- the top-k is taken before the softmax, so the kept gate values
 *   keep continuous derivatives and gradients reach the gate; "Kernideen" --
 *   the noise term keeps them smooth; "Load-Balancing-Losses").
 * Loss: L = sum(dy * y) + w_switch * aux[0] + w_importance * aux[1] +
 * w_load * aux[2] (aux as moe_route; w_load only with w_noise), with y the
 * layer output of moe_forward on the same inputs and parameters. The discrete
 * choices -- top-k sets (the canonical routing), ranks, capacity drops -- are
 * held fixed; everything else is differentiated:
 *   experts:  dW2[e] = sum over e's kept rows of act(z)^T (g dy_t),
 *             dW1[e] = sum of x_t^T dz, dz = ((g dy_t) W2[e]^T) * act'(z);
 *   gate:     dL/dg = <dy_t, expert output> (kept) + the importance term;
 *             through Softmax(KeepTopK) (renormalize = 1) or the full softmax
 *             (0, and the switch loss), the load estimator's Phi terms (its
 *             threshold's gradient goes to the expert holding kth_excluding),
 *             H = clean + noise * softplus(x W_noise);
 *   inputs:   dx_t = sum of the row gradients of its kept slots + dclean_t W_gate^T
 *             (+ du_t W_noise^T).
 * The layer is recomputed inside (routing, dispatch, both expert layers), so
 * only the forward's inputs are needed.
 * Inputs as moe_forward, plus dy [T,d] dtype and the three loss weights (host
 * doubles, finite; 0 leaves a loss out).
 * Outputs: dx [T,d] dtype; dw_gate [d,E] fp32; dgate_bias [E] fp32 (written iff
 *          gate_bias and dgate_bias are both non-NULL); dw_noise [d,E] fp32
 *          (required iff w_noise); dw1 [E,d,f] and dw2 [E,f,d] dtype (experts
 *          with no rows get zeros); dlogits [T,E] fp32 or NULL: dL/d(clean
 *          logits x W_gate + b).
 * Workspace: moe_workspace_size(p, MOE_OP_BACKWARD).
 */
moe_status moe_backward(const moe_params* p, const void* x, const void* w_gate, const float* gate_bias,
                        const void* w_noise, const float* noise, const void* w1, const void* w2, const void* dy,
                        double w_switch, double w_importance, double w_load, void* dx, float* dw_gate,
                        float* dgate_bias, float* dw_noise, void* dw1, void* dw2, float* dlogits, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * moe_set_phase_events -- phase timing of moe_forward (a measurement aid; the
 * layer's results do not depend on it).
 * After this call, every moe_forward on the calling thread records events[i]
 * (hipEvent_t handles, created by the caller) on its stream at these points:
 *   0 before the route, 1 after the route, 2 after the dispatch, 3 after the
 *   first expert layer's launch, 4 after the second expert layer's launch,
 *   5 at the end (after the combine; top-1 bf16 layers have none).
 * Entries i >= n, or NULL, are not recorded. n = 0 or events = NULL turns the
 * recording off. The library keeps the handles, not copies: the events must
 * outlive the calls that record them. Thread-local.
 * Returns MOE_ERR_INVALID_ARG unless 0 <= n <= 6.
 */
moe_status moe_set_phase_events(void* const* events, int n);

/*
 * moe_standard_normal -- the StandardNormal() noise of the noisy gate (Shazeer
 * "Methode", Noisy Top-K Gating) drawn on the device as a counter-based stream,
 * bit-identical on any machine that follows the definition:
 *   out[r][c] = N(seed, row0 + r, c), r < rows, c < cols (row-major, fp32), where
 *   N(seed, row, col): Philox4x32-10 (Salmon et al., SC 2011) of the counter
 *   (col, row & 0xFFFFFFFF, row >> 32, 0) under the key (seed & 0xFFFFFFFF,
 *   seed >> 32) gives words w0, w1; u1 = ((w0 >> 8) + 1) 2^-24, u2 = (w1 >> 8)
 *   2^-24; N = sqrt(-2 ln u1) cos(2 pi u2), with ln, cos and sqrt evaluated from
 *   correctly rounded fp32 operations (ln u = log1p(u - 1) for u >= 1/2, else
 *   e ln2 + log1p(m - 1), log1p as in moe_route's softplus; cos folded to
 *   [0, pi/4] and Taylor polynomials of degree 10 / 11).
 * Use it to fill moe_route's `noise` [T,E] (row = token, col = expert): any
 * slice of tokens can be drawn alone with its row0.
 * out: device, rows * cols fp32. Errors: MOE_ERR_INVALID_ARG for negative
 * sizes or a row range past 2^63.
 */
moe_status moe_standard_normal(uint64_t seed, int64_t row0, int64_t rows, int32_t cols, float* out, void* stream);

/*
 * moe_canonical_softplus -- the softplus of the noisy gate (Shazeer "Methode",
 * Noisy Top-K Gating: Softplus((x W_noise)_i)), element-wise, exactly as
 * moe_route evaluates it (see the definition above moe_route).
 * Inputs: z [n] fp32. Outputs: out [n] fp32. n >= 0.
 */
moe_status moe_canonical_softplus(const float* z, float* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
