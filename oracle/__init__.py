"""CPU oracle for the sparsely-gated MoE layer forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It never touches the GPU
library and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain loops, gcc, no fast-math);
this module marshals numpy arrays into it and composes the steps of the layer
in the order the pages give them:

1. gate logits (noisy top-k gating on the Shazeer et al. summary page,
   "Methode"; the linear router of the "Switch Transformer" page's listing),
2. top-k order and gate values (KeepTopK + Softmax; or Switch's raw top-1
   probability),
3. balancing losses ("Load-Balancing-Losses"; Switch's auxiliary loss),
4. capacity-limited dispatch grouped by expert,
5. each expert's two-layer FFN,
6. the gate-weighted combine y = sum_i G(x)_i E_i(x).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_LIB = None
F32, BF16 = 0, 1
RELU, GELU = 0, 1


def _lib():
    global _LIB
    if _LIB is None:
        # MOE_ORACLE_LIB: another build of moe_oracle.c (the sanitizer test loads an
        # ASan/UBSan build through it)
        path = os.environ.get("MOE_ORACLE_LIB")
        if path is None:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sigs = {
            "oracle_num_threads": ([], ctypes.c_int),
            "oracle_softplus": ([ctypes.c_float], ctypes.c_float),
            "oracle_softplus_n": ([P, P, i64], None),
            "oracle_exp_nonpos_n": ([P, P, i64], None),
            "oracle_log1p_unit_n": ([P, P, i64], None),
            "oracle_gate_logits": ([i64, i32, i32, i32, P, P, P, P, P, P, P, P], None),
            "oracle_topk_order": ([i64, i32, i32, P, P], None),
            "oracle_gates": ([i64, i32, i32, i32, P, P, P, P], None),
            "oracle_load": ([i64, i32, i32, P, P, P, P, i32, P], None),
            "oracle_aux": ([i64, i32, i32, P, P, P, P, P], None),
            "oracle_capacity": ([i64, i32, i32, dbl, i64], i64),
            "oracle_dispatch": ([i64, i32, i32, i64, i32, P, P, P, P, P, P], None),
            "oracle_expert_ffn_rows": ([i64, i32, i32, i32, i32, P, P, P, P, P, P], None),
            "oracle_combine": ([i64, P, i32, i32, P, P, P, P, P], None),
            "oracle_expert_bwd_rows": ([i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P], None),
            "oracle_philox_words": ([ctypes.c_uint64, i64, i64, i32, P], None),
            "oracle_normal_noise": ([ctypes.c_uint64, i64, i64, i32, P], None),
            "oracle_normal_from_words_n": ([P, i64, P], None),
            "oracle_gate_bwd": ([i64, i64, i32, i32, i32, P, P, P, P, P, i32, P, P, P, dbl, P, P, P], None),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _wdtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def _dcode(dtype: str) -> int:
    return BF16 if dtype == "bf16" else F32


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


# --------------------------------------------------------------------------
# canonical softplus and its two pieces (fp32)
# --------------------------------------------------------------------------
def softplus(z) -> np.ndarray:
    z = _c(np.atleast_1d(z), np.float32)
    out = np.empty_like(z)
    _lib().oracle_softplus_n(_p(z), _p(out), z.size)
    return out


def exp_nonpos(y) -> np.ndarray:
    y = _c(np.atleast_1d(y), np.float32)
    out = np.empty_like(y)
    _lib().oracle_exp_nonpos_n(_p(y), _p(out), y.size)
    return out


def log1p_unit(v) -> np.ndarray:
    v = _c(np.atleast_1d(v), np.float32)
    out = np.empty_like(v)
    _lib().oracle_log1p_unit_n(_p(v), _p(out), v.size)
    return out


# --------------------------------------------------------------------------
# steps
# --------------------------------------------------------------------------
def gate_logits(x, w_gate, gate_bias=None, w_noise=None, noise=None, dtype="bf16"):
    """Canonical fp32 logits. Returns (clean, sigma or None, H), each [T,E] float32."""
    wd = _wdtype(dtype)
    x = _c(x, wd)
    w_gate = _c(w_gate, wd)
    T, d = x.shape
    E = w_gate.shape[1]
    assert w_gate.shape[0] == d
    gate_bias = _c(gate_bias, np.float32)
    noisy = w_noise is not None
    w_noise = _c(w_noise, wd)
    noise = _c(noise, np.float32)
    clean = np.empty((T, E), np.float32)
    H = np.empty((T, E), np.float32)
    sigma = np.empty((T, E), np.float32) if noisy else None
    _lib().oracle_gate_logits(T, d, E, _dcode(dtype), _p(x), _p(w_gate), _p(gate_bias), _p(w_noise),
                              _p(noise), _p(clean), _p(sigma), _p(H))
    return clean, sigma, H


def topk_order(H, kk: int) -> np.ndarray:
    H = _c(H, np.float32)
    T, E = H.shape
    out = np.empty((T, kk), np.int32)
    _lib().oracle_topk_order(T, E, kk, _p(H), _p(out))
    return out


def gates(H, topk_idx, renormalize: bool, want_prob: bool = True):
    H = _c(H, np.float32)
    idx = _c(topk_idx, np.int32)
    T, E = H.shape
    k = idx.shape[1]
    g = np.empty((T, k), np.float64)
    prob = np.empty((T, E), np.float64) if want_prob else None
    _lib().oracle_gates(T, E, k, int(bool(renormalize)), _p(H), _p(idx), _p(g), _p(prob))
    return g, prob


def load(clean, sigma, H, order, k: int) -> np.ndarray:
    clean, sigma, H = (_c(a, np.float32) for a in (clean, sigma, H))
    order = _c(order, np.int32)
    T, E = H.shape
    out = np.empty(E, np.float64)
    _lib().oracle_load(T, E, k, _p(clean), _p(sigma), _p(H), _p(order), order.shape[1], _p(out))
    return out


def aux(T: int, k: int, counts_routed, prob_sum, importance, load_vec=None) -> np.ndarray:
    counts_routed = _c(counts_routed, np.int32)
    E = counts_routed.shape[0]
    prob_sum = _c(prob_sum, np.float64)
    importance = _c(importance, np.float64)
    load_vec = _c(load_vec, np.float64)
    out = np.empty(3, np.float64)
    _lib().oracle_aux(T, E, k, _p(counts_routed), _p(prob_sum), _p(importance), _p(load_vec), _p(out))
    return out


def capacity(T: int, E: int, k: int, capacity_factor: float, explicit: int = -1) -> int:
    """Per-expert capacity, or -1 for no limit."""
    return int(_lib().oracle_capacity(T, E, k, float(capacity_factor), int(explicit)))


def dispatch(topk_idx, E: int, C: int, slot_major: bool = False) -> dict:
    """Capacity-limited dispatch. slot_major=False: overflow dropped in token order;
    True: first-choice priority (all first choices ranked before any second choice)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts_routed = np.empty(E, np.int32)
    counts_kept = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot_dest = np.empty((T, k), np.int32)
    row_src = np.full(max(T * k, 1), -1, np.int32)
    _lib().oracle_dispatch(T, E, k, int(C), int(bool(slot_major)), _p(idx), _p(counts_routed), _p(counts_kept),
                           _p(offsets), _p(slot_dest), _p(row_src))
    R = int(offsets[E])
    return dict(counts_routed=counts_routed, counts_kept=counts_kept, offsets=offsets,
                slot_dest=slot_dest, row_src=row_src[:R].copy(), R=R)


def expert_ffn_rows(x, x_row, expert, w1, w2, act: str, dtype: str) -> np.ndarray:
    """fp64 FFN output of expert[r] applied to x[x_row[r]], for each r."""
    wd = _wdtype(dtype)
    x = _c(x, wd)
    w1 = _c(w1, wd)
    w2 = _c(w2, wd)
    x_row = _c(x_row, np.int32)
    expert = _c(expert, np.int32)
    n = x_row.shape[0]
    d = x.shape[1]
    f = w1.shape[2]
    assert w1.shape[1] == d and w2.shape[1] == f and w2.shape[2] == d
    out = np.empty((n, d), np.float64)
    if n:
        _lib().oracle_expert_ffn_rows(n, d, f, _dcode(dtype), RELU if act == "relu" else GELU, _p(x),
                                      _p(x_row), _p(expert), _p(w1), _p(w2), _p(out))
    return out


def combine(tokens, slot_dest, gate_vals, yp, yp_row_of_slot=None) -> np.ndarray:
    tokens = _c(tokens, np.int32)
    slot_dest = _c(slot_dest, np.int32)
    gate_vals = _c(gate_vals, np.float64)
    yp = _c(yp, np.float64)
    k = slot_dest.shape[1]
    d = yp.shape[1]
    rows = _c(yp_row_of_slot, np.int32)
    y = np.empty((tokens.shape[0], d), np.float64)
    _lib().oracle_combine(tokens.shape[0], _p(tokens), d, k, _p(slot_dest), _p(gate_vals), _p(yp),
                          _p(rows), _p(y))
    return y


# --------------------------------------------------------------------------
# composed layer
# --------------------------------------------------------------------------
@dataclass
class LayerSpec:
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    dtype: str
    act: str
    renormalize: bool
    capacity_factor: float = 0.0
    capacity: int = -1  # explicit per-expert capacity; -1 derives it from the factor
    slot_major: bool = False  # drop order: False = token order, True = first-choice priority

    @classmethod
    def of(cls, cfg, capacity: int = -1, slot_major: bool = False) -> "LayerSpec":
        return cls(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, bool(cfg.renormalize),
                   float(cfg.capacity_factor), int(capacity), bool(slot_major))


def route(spec: LayerSpec, inp: dict) -> dict:
    """Gate logits, top-k, gate values, per-expert routed counts and the losses."""
    clean, sigma, H = gate_logits(inp["x"], inp["w_gate"], inp.get("gate_bias"), inp.get("w_noise"),
                                  inp.get("noise"), spec.dtype)
    T, E, k = spec.T, spec.E, spec.k
    noisy = inp.get("w_noise") is not None
    kk = min(k + 1, E) if noisy else k
    order = topk_order(H, kk)
    topk_idx = np.ascontiguousarray(order[:, :k])
    g, prob = gates(H, topk_idx, spec.renormalize)
    counts_routed = np.bincount(topk_idx.ravel(), minlength=E).astype(np.int32)
    importance = np.zeros(E, np.float64)
    np.add.at(importance, topk_idx.ravel(), g.ravel())
    ld = load(clean, sigma, H, order, k) if noisy else None
    a = aux(T, k, counts_routed, prob.sum(axis=0), importance, ld)
    return dict(clean=clean, sigma=sigma, H=H, order=order, topk_idx=topk_idx, topk_gate=g, prob=prob,
                counts_routed=counts_routed, importance=importance, load=ld, aux=a)


def forward(spec: LayerSpec, inp: dict, tokens=None) -> dict:
    """The whole layer. ``tokens`` (optional) restricts the expert FFN and the
    combine to those tokens (routing and dispatch always cover the batch);
    ``y`` then holds one row per listed token, in the listed order."""
    r = route(spec, inp)
    C = capacity(spec.T, spec.E, spec.k, spec.capacity_factor, spec.capacity)
    disp = dispatch(r["topk_idx"], spec.E, C, spec.slot_major)
    out = dict(r)
    out.update(disp)
    out.update(_experts_and_combine(spec, inp, r["topk_idx"], r["topk_gate"], disp, tokens))
    out.update(C=C)
    return out


def _experts_and_combine(spec, inp, topk_idx, topk_gate, disp, tokens):
    """Each kept assignment's expert FFN output, gate-weighted and summed per token."""
    T, k = spec.T, topk_idx.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.asarray(tokens, dtype=np.int32)
    slots = disp["slot_dest"][tokens]  # [n, k]
    kept = slots >= 0
    rows_slot = slots[kept]
    rows_tok = np.repeat(tokens, k).reshape(-1, k)[kept]
    rows_exp = topk_idx[tokens][kept]
    yp = expert_ffn_rows(inp["x"], rows_tok, rows_exp, inp["w1"], inp["w2"], spec.act, spec.dtype)
    R = disp["R"]
    row_of_slot = np.full(max(R, 1), -1, np.int32)
    row_of_slot[rows_slot] = np.arange(rows_slot.shape[0], dtype=np.int32)
    y = combine(tokens, disp["slot_dest"], topk_gate, yp if yp.size else np.zeros((1, spec.d_model)), row_of_slot)
    return dict(tokens=tokens, y=y, yp=yp, yp_slots=rows_slot)


# --------------------------------------------------------------------------
# hierarchical MoE (Shazeer et al. summary page, "Schluesselbegriffe": a primary
# gating network routes each input to secondary MoE groups; "moe paper models"
# table 2: k = 2 for the hierarchical models). Reading: the layer is a MoE of
# MoEs, y = sum_i Gp(x)_i sum_j G_i(x)_j E_ij(x), each gate a (noisy) top-k gate
# of the "Methode" section with the softmax over its kept logits; the expert
# slots of a token are (kept group r, kept expert q of that group) in that order,
# expert id i * b + j, gate Gp_i * G_i,j. Losses: CV^2 of the primary importance
# (per group), CV^2 of the importance of the combined gates (per expert), CV^2 of
# the primary load (noisy primary gate; else NaN).
# --------------------------------------------------------------------------
@dataclass
class HierSpec:
    T: int
    d_model: int
    d_ff: int
    groups: int
    experts_per_group: int
    k_group: int
    k: int
    dtype: str
    act: str
    capacity_factor: float = 0.0
    capacity: int = -1

    @property
    def E(self) -> int:
        return self.groups * self.experts_per_group

    @property
    def slots(self) -> int:
        return self.k_group * self.k

    @classmethod
    def of(cls, cfg, capacity: int = -1) -> "HierSpec":
        return cls(cfg.T, cfg.d_model, cfg.d_ff, cfg.groups, cfg.experts_per_group, cfg.k_group, cfg.k, cfg.dtype,
                   cfg.act, float(cfg.capacity_factor), int(capacity))


def route_hier(spec: HierSpec, inp: dict) -> dict:
    T, a, b, kp, ks, E = spec.T, spec.groups, spec.experts_per_group, spec.k_group, spec.k, spec.E
    clean_p, sig_p, Hp = gate_logits(inp["x"], inp["w_gate_p"], inp.get("gate_bias_p"), inp.get("w_noise_p"),
                                     inp.get("noise_p"), spec.dtype)
    clean_s, sig_s, Hs = gate_logits(inp["x"], inp["w_gate_s"], inp.get("gate_bias_s"), inp.get("w_noise_s"),
                                     inp.get("noise_s"), spec.dtype)
    noisy_p = inp.get("w_noise_p") is not None
    order_p = topk_order(Hp, min(kp + 1, a) if noisy_p else kp)
    top_p = np.ascontiguousarray(order_p[:, :kp])
    gp, _ = gates(Hp, top_p, True, want_prob=False)
    # each kept group's own top-k over its b experts, softmax over the kept logits
    Hsel = np.ascontiguousarray(Hs.reshape(T, a, b)[np.arange(T)[:, None], top_p].reshape(T * kp, b))
    js = topk_order(Hsel, ks)
    gs, _ = gates(Hsel, js, True, want_prob=False)
    topk_idx = (top_p[:, :, None] * b + js.reshape(T, kp, ks)).reshape(T, kp * ks).astype(np.int32)
    topk_gate = (gp[:, :, None] * gs.reshape(T, kp, ks)).reshape(T, kp * ks)
    counts_routed = np.bincount(topk_idx.ravel(), minlength=E).astype(np.int32)
    imp_p = np.zeros(a, np.float64)
    np.add.at(imp_p, top_p.ravel(), gp.ravel())
    imp_c = np.zeros(E, np.float64)
    np.add.at(imp_c, topk_idx.ravel(), topk_gate.ravel())
    load_p = load(clean_p, sig_p, Hp, order_p, kp) if noisy_p else None
    counts_p = np.bincount(top_p.ravel(), minlength=a).astype(np.int32)
    a_p = aux(T, kp, counts_p, np.zeros(a), imp_p, load_p)
    a_c = aux(T, kp * ks, counts_routed, np.zeros(E), imp_c)
    return dict(Hp=Hp, Hs=Hs, clean_p=clean_p, sigma_p=sig_p, order_p=order_p, gate_p=gp, topk_idx=topk_idx,
                topk_gate=topk_gate, counts_routed=counts_routed, importance_p=imp_p, importance=imp_c,
                load_p=load_p, aux=np.array([a_p[1], a_c[1], a_p[2]]))


def forward_hier(spec: HierSpec, inp: dict, tokens=None) -> dict:
    r = route_hier(spec, inp)
    C = capacity(spec.T, spec.E, spec.slots, spec.capacity_factor, spec.capacity)
    disp = dispatch(r["topk_idx"], spec.E, C)
    out = dict(r)
    out.update(disp)
    out.update(_experts_and_combine(spec, inp, r["topk_idx"], r["topk_gate"], disp, tokens))
    out.update(C=C)
    return out


# --------------------------------------------------------------------------
# backward pass (the pages train the layer: Shazeer et al. summary page,
# "Fragen" -- gradients flow through the kept gates because the top-k is taken
# before the softmax; "Kernideen" -- the noise term keeps them smooth)
# --------------------------------------------------------------------------
def expert_bwd_rows(x, x_row, expert, w1, w2, dout, act: str, dtype: str, want_dw: bool = True):
    """fp64 expert FFN backward for rows r (expert[r] applied to x[x_row[r]])
    with upstream gradient dout[r]. Returns (o, dx_rows, dw1, dw2); dw1 / dw2
    are None with want_dw=False."""
    wd = _wdtype(dtype)
    x, w1, w2 = _c(x, wd), _c(w1, wd), _c(w2, wd)
    x_row, expert = _c(x_row, np.int32), _c(expert, np.int32)
    dout = _c(dout, np.float64)
    n, d = dout.shape
    E, _, f = w1.shape
    o = np.zeros((n, d), np.float64)
    dx_rows = np.zeros((n, d), np.float64)
    dw1 = np.empty((E, d, f), np.float64) if want_dw else None
    dw2 = np.empty((E, f, d), np.float64) if want_dw else None
    _lib().oracle_expert_bwd_rows(n, d, f, E, _dcode(dtype), RELU if act == "relu" else GELU, _p(x), _p(x_row),
                                  _p(expert), _p(w1), _p(w2), _p(dout), _p(o), _p(dx_rows), _p(dw1), _p(dw2))
    return o, dx_rows, dw1, dw2


def gate_bwd(H, clean, sigma, noise, order, k: int, renormalize: bool, g, dg, counts_routed, w_switch: float,
             dload=None, T_batch=None):
    """dL/dclean [T,E] and (noisy) dL/d(x W_noise) [T,E], fp64. The rows may be a
    subset of a batch of T_batch tokens."""
    H, clean = _c(H, np.float32), _c(clean, np.float32)
    sigma, noise = _c(sigma, np.float32), _c(noise, np.float32)
    order = _c(order, np.int32)
    g, dg = _c(g, np.float64), _c(dg, np.float64)
    counts_routed = _c(counts_routed, np.int32)
    dload = _c(dload, np.float64)
    T, E = H.shape
    dclean = np.empty((T, E), np.float64)
    du = np.empty((T, E), np.float64) if sigma is not None else None
    _lib().oracle_gate_bwd(T, int(T if T_batch is None else T_batch), E, k, int(bool(renormalize)), _p(H), _p(clean),
                           _p(sigma), _p(noise), _p(order),
                           order.shape[1], _p(g), _p(dg), _p(counts_routed), float(w_switch), _p(dload),
                           _p(dclean), _p(du))
    return dclean, du


def cv2_grad(v) -> np.ndarray:
    """d CV(v)^2 / dv for the population CV (Load-Balancing-Losses); 0 for one entry."""
    v = np.asarray(v, np.float64)
    E = v.size
    if E <= 1:
        return np.zeros_like(v)
    mu = v.sum() / E
    var = ((v - mu) ** 2).sum() / E
    return 2.0 * (v - mu) / (E * mu * mu) - 2.0 * var / (E * mu ** 3)


def backward(spec: LayerSpec, inp: dict, dy, loss_weights=(0.0, 0.0, 0.0), tokens=None, experts=None) -> dict:
    """Gradients of L = sum(dy * y) + w_switch * switch_aux + w_importance *
    CV(Importance)^2 + w_load * CV(Load)^2 with respect to x, W_gate, gate_bias,
    W_noise, W1 and W2, with the layer's discrete choices (top-k sets, capacity
    drops) held fixed. fp64 throughout (logits: the forward's canonical fp32).

    ``tokens`` / ``experts`` (optional) restrict the work for large batches: the
    expert FFN is evaluated only on the kept rows of the listed tokens and all
    rows of the listed experts; dx, dclean and du then hold one row per listed
    token, dw1 / dw2 map each listed expert to its gradients, and the gate weight
    gradients (which need every token) are not formed. Routing, dispatch and
    the batch statistics of the losses always cover the whole batch."""
    w_switch, w_imp, w_load = (float(w) for w in loss_weights)
    r = route(spec, inp)
    C = capacity(spec.T, spec.E, spec.k, spec.capacity_factor, spec.capacity)
    disp = dispatch(r["topk_idx"], spec.E, C, spec.slot_major)
    T, k, E = spec.T, spec.k, spec.E
    subset = tokens is not None or experts is not None
    tok_sel = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    dy = np.asarray(dy, np.float64)
    kept = disp["slot_dest"] >= 0
    tok = np.repeat(np.arange(T, dtype=np.int32), k).reshape(T, k)
    want = np.zeros((T, k), bool)
    want[tok_sel] = True
    if experts is not None:
        want |= np.isin(r["topk_idx"], np.asarray(experts))
    use = kept & want if subset else kept
    rows_tok, rows_exp = tok[use], r["topk_idx"][use]
    g = r["topk_gate"]
    dout = g[use][:, None] * dy[rows_tok]
    o, dx_rows, dw1, dw2 = expert_bwd_rows(inp["x"], rows_tok, rows_exp, inp["w1"], inp["w2"], dout, spec.act,
                                           spec.dtype, want_dw=not subset)
    if subset and experts is not None:
        # weight gradients of the listed experts only, one expert at a time
        dw1, dw2 = {}, {}
        for e in np.asarray(experts):
            m = use & (r["topk_idx"] == e)
            _, _, a1, a2 = expert_bwd_rows(inp["x"], tok[m], np.zeros(int(m.sum()), np.int32),
                                           inp["w1"][e:e + 1], inp["w2"][e:e + 1],
                                           g[m][:, None] * dy[tok[m]], spec.act, spec.dtype)
            dw1[int(e)], dw2[int(e)] = a1[0], a2[0]
    # dL/dg: the combine (kept slots only) plus the importance loss (all slots, pre-drop)
    dg = np.zeros((T, k), np.float64)
    dg[use] = np.einsum("rd,rd->r", dy[rows_tok], o)
    if w_imp:
        dg += w_imp * cv2_grad(r["importance"])[r["topk_idx"]]
    noisy = inp.get("w_noise") is not None
    dload = w_load * cv2_grad(r["load"]) if (noisy and w_load) else None
    sel = lambda a: None if a is None else np.ascontiguousarray(a[tok_sel])  # noqa: E731
    dclean, du = gate_bwd(sel(r["H"]), sel(r["clean"]), sel(r["sigma"]), sel(inp.get("noise")), sel(r["order"]), k,
                          spec.renormalize, sel(g), sel(dg), r["counts_routed"], w_switch, dload, T_batch=T)
    xf = bf16_widen(inp["x"]) if spec.dtype == "bf16" else np.asarray(inp["x"], np.float64)
    wg = bf16_widen(inp["w_gate"]) if spec.dtype == "bf16" else np.asarray(inp["w_gate"], np.float64)
    dx_all = np.zeros((T, spec.d_model), np.float64)
    np.add.at(dx_all, rows_tok, dx_rows)
    dx = dx_all[tok_sel] + dclean @ wg.T
    out = dict(dx=dx, dw1=dw1, dw2=dw2, dg=dg, dclean=dclean, o=o, route=r, disp=disp, du=du, tokens=tok_sel,
               dw_gate=None, dgate_bias=None, dw_noise=None)
    if noisy:
        wn = bf16_widen(inp["w_noise"]) if spec.dtype == "bf16" else np.asarray(inp["w_noise"], np.float64)
        dx += du @ wn.T
    out["dx"] = dx
    if not subset:
        out["dw_gate"] = xf.T @ dclean
        if inp.get("gate_bias") is not None:
            out["dgate_bias"] = dclean.sum(axis=0)
        if noisy:
            out["dw_noise"] = xf.T @ du
    return out


def bf16_widen(a) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.ascontiguousarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# counter-based standard-normal noise (Shazeer et al. summary page, "Noisy
# Top-K Gating": StandardNormal()); see moe_oracle.c for the definition
# --------------------------------------------------------------------------
def philox_words(seed: int, rows: int, cols: int, row0: int = 0) -> np.ndarray:
    """Philox4x32-10 output words [rows, cols, 4] of counters (col, row lo, row hi, 0)."""
    out = np.empty((rows, cols, 4), np.uint32)
    _lib().oracle_philox_words(int(seed), int(row0), int(rows), int(cols), _p(out))
    return out


def normal_noise(seed: int, rows: int, cols: int, row0: int = 0) -> np.ndarray:
    """Standard normals [rows, cols] fp32: Box-Muller on the first two Philox words."""
    out = np.empty((rows, cols), np.float32)
    _lib().oracle_normal_noise(int(seed), int(row0), int(rows), int(cols), _p(out))
    return out


def normal_from_words(words) -> np.ndarray:
    """The transform alone: words [..., 2] uint32 -> standard normals fp32."""
    w = np.ascontiguousarray(words, np.uint32).reshape(-1, 2)
    out = np.empty(w.shape[0], np.float32)
    _lib().oracle_normal_from_words_n(_p(w), w.shape[0], _p(out))
    return out
