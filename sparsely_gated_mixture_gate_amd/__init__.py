"""Python binding of ``libmoe.so``, the gfx950 sparsely-gated MoE layer forward.

Thin ctypes marshalling over the C ABI in ``include/moe.h``: each function
here has the name of the C entry point it calls, takes torch tensors (device
memory) and passes their pointers and the current HIP stream. Every step of
the layer runs in the library's HIP kernels; nothing here computes. If the
library is missing, the first call raises -- there is no fallback. The
library is loaded on first use, not at import, so the package (and its build
module) can be imported before anything is built.

Build the library with ``python -m sparsely_gated_mixture_gate_amd.build`` or
``__graft_entry__.build()``.
"""

from __future__ import annotations

import ctypes
import os

# MOE_LIB names another build of the same library (the host-sanitizer test loads an
# AddressSanitizer build through it); by default the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_RELU, MOE_ACT_GELU = 0, 1
(MOE_OP_ROUTE, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_FORWARD, MOE_OP_BACKWARD, MOE_OP_ROUTE_HIER,
 MOE_OP_FORWARD_HIER) = range(7)
MOE_GATE_AUTO, MOE_GATE_CANONICAL, MOE_GATE_FALLBACK, MOE_GATE_EXPORT = range(4)
MOE_DROP_TOKEN_ORDER, MOE_DROP_FIRST_CHOICE = range(2)

EXPORTED = (
    "moe_status_string", "moe_last_error", "moe_capacity", "moe_max_rows", "moe_workspace_size",
    "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_canonical_softplus",
    "moe_set_phase_events", "moe_dispatch_noalloc", "moe_backward", "moe_route_hier", "moe_forward_hier",
    "moe_standard_normal",
)


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)}: {detail}")
        self.status = status


class moe_params(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("gate_mode", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("capacity", ctypes.c_int64),
        ("drop_order", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("k_group", ctypes.c_int32),
    ]


_LIB = None


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    # torch ships its own HIP runtime (soname libamdhip64.so.7). Loading torch
    # first makes libmoe.so bind to that same runtime instance, so the library
    # and torch share one device context, its streams and its allocations.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(moe_params)
    sz, i64, i32 = ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    sigs = {
        "moe_status_string": ([i32], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_capacity": ([PP], i64),
        "moe_max_rows": ([PP], i64),
        "moe_workspace_size": ([PP, i32, ctypes.POINTER(sz)], i32),
        "moe_route": ([PP, P, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "moe_dispatch": ([PP, P, P, P, P, P, P, P, P, sz, P], i32),
        "moe_expert_ffn": ([PP, P, P, P, P, P, P, sz, P], i32),
        "moe_combine": ([PP, P, P, P, P, P], i32),
        "moe_forward": ([PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "moe_canonical_softplus": ([P, P, i64, P], i32),
        "moe_set_phase_events": ([ctypes.POINTER(P), i32], i32),
        "moe_dispatch_noalloc": ([PP, P, P, P, P, P, P, P, P], i32),
        "moe_standard_normal": ([ctypes.c_uint64, i64, i64, i32, P, P], i32),
        "moe_route_hier": ([PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "moe_forward_hier": ([PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "moe_backward": ([PP, P, P, P, P, P, P, P, P, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                          P, P, P, P, P, P, P, P, sz, P], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def lib() -> ctypes.CDLL:
    """The loaded ``libmoe.so`` (loaded on the first call; raises if it is not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoEError(st, where, lib().moe_last_error().decode())


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def make_params(T, d_model, d_ff, E, k, dtype="bf16", act="gelu", renormalize=False, capacity_factor=0.0,
                capacity=-1, gate_mode=0, drop_order=0, groups=0, k_group=0) -> moe_params:
    return moe_params(int(T), int(d_model), int(d_ff), int(E), int(k),
                      MOE_BF16 if dtype in ("bf16", MOE_BF16) else MOE_F32,
                      MOE_ACT_GELU if act in ("gelu", MOE_ACT_GELU) else MOE_ACT_RELU,
                      int(bool(renormalize)), int(gate_mode), float(capacity_factor), int(capacity),
                      int(drop_order), int(groups), int(k_group))


def moe_capacity(p: moe_params) -> int:
    return int(lib().moe_capacity(ctypes.byref(p)))


def moe_max_rows(p: moe_params) -> int:
    return int(lib().moe_max_rows(ctypes.byref(p)))


def moe_workspace_size(p: moe_params, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(p), int(op), ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------
def moe_route(p, x, w_gate, gate_bias, w_noise, noise, topk_idx, topk_gate, counts_routed, aux_out=None,
              logits_out=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(gate_bias), _ptr(w_noise), _ptr(noise),
                          _ptr(topk_idx), _ptr(topk_gate), _ptr(counts_routed), _ptr(aux_out), _ptr(logits_out),
                          wp, wn, _stream(stream)), "moe_route")


def moe_dispatch(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_dispatch(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(counts_kept), _ptr(offsets),
                             _ptr(slot_dest), _ptr(row_src), _ptr(x_perm), wp, wn, _stream(stream)), "moe_dispatch")


def moe_dispatch_noalloc(p, x, topk_idx, counts_kept, offsets, slot_dest, row_src, x_perm, stream=None):
    _check(lib().moe_dispatch_noalloc(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(counts_kept), _ptr(offsets),
                                      _ptr(slot_dest), _ptr(row_src), _ptr(x_perm), _stream(stream)),
           "moe_dispatch_noalloc")


def moe_expert_ffn(p, x_perm, offsets, w1, w2, y_perm, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w2), _ptr(y_perm),
                               wp, wn, _stream(stream)), "moe_expert_ffn")


def moe_combine(p, y_perm, slot_dest, topk_gate, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(slot_dest), _ptr(topk_gate), _ptr(y),
                            _stream(stream)), "moe_combine")


def moe_forward(p, x, w_gate, gate_bias, w_noise, noise, w1, w2, y, aux_out=None, topk_idx=None, topk_gate=None,
                counts_routed=None, counts_kept=None, slot_dest=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(gate_bias), _ptr(w_noise), _ptr(noise),
                            _ptr(w1), _ptr(w2), _ptr(y), _ptr(aux_out), _ptr(topk_idx), _ptr(topk_gate),
                            _ptr(counts_routed), _ptr(counts_kept), _ptr(slot_dest), wp, wn, _stream(stream)),
           "moe_forward")


def moe_route_hier(p, x, w_gate_p, gate_bias_p, w_noise_p, noise_p, w_gate_s, gate_bias_s, w_noise_s, noise_s,
                   topk_idx, topk_gate, counts_routed, aux_out=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_route_hier(ctypes.byref(p), _ptr(x), _ptr(w_gate_p), _ptr(gate_bias_p), _ptr(w_noise_p),
                                _ptr(noise_p), _ptr(w_gate_s), _ptr(gate_bias_s), _ptr(w_noise_s), _ptr(noise_s),
                                _ptr(topk_idx), _ptr(topk_gate), _ptr(counts_routed), _ptr(aux_out), wp, wn,
                                _stream(stream)), "moe_route_hier")


def moe_forward_hier(p, x, w_gate_p, gate_bias_p, w_noise_p, noise_p, w_gate_s, gate_bias_s, w_noise_s, noise_s,
                     w1, w2, y, aux_out=None, topk_idx=None, topk_gate=None, counts_routed=None, counts_kept=None,
                     slot_dest=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward_hier(ctypes.byref(p), _ptr(x), _ptr(w_gate_p), _ptr(gate_bias_p), _ptr(w_noise_p),
                                  _ptr(noise_p), _ptr(w_gate_s), _ptr(gate_bias_s), _ptr(w_noise_s), _ptr(noise_s),
                                  _ptr(w1), _ptr(w2), _ptr(y), _ptr(aux_out), _ptr(topk_idx), _ptr(topk_gate),
                                  _ptr(counts_routed), _ptr(counts_kept), _ptr(slot_dest), wp, wn, _stream(stream)),
           "moe_forward_hier")


def moe_backward(p, x, w_gate, gate_bias, w_noise, noise, w1, w2, dy, loss_weights, dx, dw_gate, dgate_bias,
                 dw_noise, dw1, dw2, dlogits=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    ws_, wi, wl = (float(v) for v in loss_weights)
    _check(lib().moe_backward(ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(gate_bias), _ptr(w_noise), _ptr(noise),
                              _ptr(w1), _ptr(w2), _ptr(dy), ws_, wi, wl, _ptr(dx), _ptr(dw_gate), _ptr(dgate_bias),
                              _ptr(dw_noise), _ptr(dw1), _ptr(dw2), _ptr(dlogits), wp, wn, _stream(stream)),
           "moe_backward")


def moe_standard_normal(seed, rows, cols, out, row0=0, stream=None):
    _check(lib().moe_standard_normal(int(seed), int(row0), int(rows), int(cols), _ptr(out), _stream(stream)),
           "moe_standard_normal")


def moe_canonical_softplus(z, out, stream=None):
    _check(lib().moe_canonical_softplus(_ptr(z), _ptr(out), int(z.numel()), _stream(stream)),
           "moe_canonical_softplus")


def moe_set_phase_events(events=None):
    """Record torch.cuda.Event objects at the phase boundaries of later
    moe_forward calls on this thread (see include/moe.h); None turns it off.
    The events must outlive those calls."""
    if not events:
        _check(lib().moe_set_phase_events(None, 0), "moe_set_phase_events")
        return
    handles = []
    for ev in events:
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            ev.record()  # the runtime creates the event on its first record
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib().moe_set_phase_events(arr, len(handles)), "moe_set_phase_events")
