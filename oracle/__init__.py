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
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
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
            "oracle_dispatch": ([i64, i32, i32, i64, P, P, P, P, P, P], None),
            "oracle_expert_ffn_rows": ([i64, i32, i32, i32, i32, P, P, P, P, P, P], None),
            "oracle_combine": ([i64, P, i32, i32, P, P, P, P, P], None),
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


def dispatch(topk_idx, E: int, C: int) -> dict:
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts_routed = np.empty(E, np.int32)
    counts_kept = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot_dest = np.empty((T, k), np.int32)
    row_src = np.full(max(T * k, 1), -1, np.int32)
    _lib().oracle_dispatch(T, E, k, int(C), _p(idx), _p(counts_routed), _p(counts_kept), _p(offsets),
                           _p(slot_dest), _p(row_src))
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

    @classmethod
    def of(cls, cfg, capacity: int = -1) -> "LayerSpec":
        return cls(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, bool(cfg.renormalize),
                   float(cfg.capacity_factor), int(capacity))


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
    disp = dispatch(r["topk_idx"], spec.E, C)
    T, k = spec.T, spec.k
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.asarray(tokens, dtype=np.int32)
    slots = disp["slot_dest"][tokens]  # [n, k]
    kept = slots >= 0
    rows_slot = slots[kept]
    rows_tok = np.repeat(tokens, k).reshape(-1, k)[kept]
    rows_exp = r["topk_idx"][tokens][kept]
    yp = expert_ffn_rows(inp["x"], rows_tok, rows_exp, inp["w1"], inp["w2"], spec.act, spec.dtype)
    R = disp["R"]
    row_of_slot = np.full(max(R, 1), -1, np.int32)
    row_of_slot[rows_slot] = np.arange(rows_slot.shape[0], dtype=np.int32)
    y = combine(tokens, disp["slot_dest"], r["topk_gate"], yp if yp.size else np.zeros((1, spec.d_model)),
                row_of_slot)
    out = dict(r)
    out.update(disp)
    out.update(C=C, tokens=tokens, y=y, yp=yp, yp_slots=rows_slot)
    return out
