"""Seeded input generators (numpy only).

Recipe: ``numpy.random.Generator(PCG64(s))`` for ``s`` in
``SeedSequence(seed).spawn(6)``, one stream per tensor in the fixed order
x, W_gate, W_noise, noise, W1, W2. W1 and W2 use one child stream per expert
(``s.spawn(E)``), so experts are drawn in parallel threads with a result that
does not depend on the thread count. Each tensor is drawn as float32 standard
normals, scaled by its standard deviation, and, for bf16 workloads, rounded to
bf16 with round-to-nearest-even. bf16 tensors are returned as ``uint16`` bit
patterns.
"""

from __future__ import annotations

import concurrent.futures as cf
import functools
import os

import numpy as np
from scipy.special import log_ndtr

from .configs import MoEConfig


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(gen: np.random.Generator, shape, std: float, dtype: str, out=None) -> np.ndarray:
    a = gen.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype != "bf16":
        if out is not None:
            out[...] = a
            return out
        return a
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    if out is not None:
        out[...] = u
        return out
    return u.astype(np.uint16)


def _expert_stack(seq: np.random.SeedSequence, E: int, shape, std: float, dtype: str) -> np.ndarray:
    st = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((E, *shape), dtype=st)
    children = seq.spawn(E)

    def one(e):
        _normal(np.random.Generator(np.random.PCG64(children[e])), shape, std, dtype, out=out[e])

    workers = max(1, min(16, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(E)))
    return out


@functools.lru_cache(maxsize=8)
def zipf_gate_bias(E: int, s: float = 1.2, logit_std: float = 1.0, iters: int = 25) -> np.ndarray:
    """Per-expert logit offsets under which top-1 shares follow Zipf(s).

    Model of the clean logits: ``b_e + logit_std * z_e`` with independent standard
    normal ``z_e`` (true to first order for x ~ N(0,1) and independent W_gate
    columns of variance 1/d). The share of expert e is
    ``P_e = integral phi(u) * prod_{j != e} Phi(u + (b_e - b_j)/logit_std) du``;
    a damped fixed-point iteration on ``log P_e`` moves it to ``(e+1)^-s``
    normalised (total-variation error below 1e-9 after 25 steps at E=64).
    Deterministic: no random numbers are drawn here.
    """
    target = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    target /= target.sum()
    u = np.linspace(-9.0, 9.0, 1201)
    du = u[1] - u[0]
    log_phi = -0.5 * u * u - 0.5 * np.log(2 * np.pi)
    idx = np.arange(E)
    b = 0.5 * np.log(target)
    b -= b.max()
    for _ in range(iters):
        diff = (b[:, None] - b[None, :]) / logit_std  # [e, j]
        lp = log_ndtr(u[None, None, :] + diff[:, :, None])  # log Phi, [e, j, U]
        lp[idx, idx, :] = 0.0
        share = np.exp(log_phi[None, :] + lp.sum(axis=1)).sum(axis=1) * du
        share = share / share.sum()
        b = b + 0.5 * (np.log(target) - np.log(share))
        b -= b.max()
    b = b.astype(np.float32)
    b.setflags(write=False)
    return b


def make_inputs(cfg: MoEConfig, seed: int = 0, with_weights: bool = True) -> dict:
    """All inputs of one layer forward for ``cfg``.

    Returns a dict with ``x [T,d]``, ``w_gate [d,E]``, ``w_noise [d,E]`` or None,
    ``noise [T,E]`` float32 or None, ``gate_bias [E]`` float32 or None,
    ``w1 [E,d,f]`` and ``w2 [E,f,d]`` (omitted when ``with_weights`` is False).
    bf16 tensors are uint16 bit patterns; f32 tensors are float32.
    """
    T, d, f, E = cfg.T, cfg.d_model, cfg.d_ff, cfg.E
    ss = np.random.SeedSequence(seed).spawn(6)
    g_x, g_wg, g_wn, g_eps = (np.random.Generator(np.random.PCG64(s)) for s in ss[:4])
    out: dict = {}
    out["x"] = _normal(g_x, (T, d), cfg.x_std, cfg.dtype)
    out["w_gate"] = _normal(g_wg, (d, E), cfg.wg_std, cfg.dtype)
    if cfg.noisy:
        out["w_noise"] = _normal(g_wn, (d, E), cfg.wn_std, cfg.dtype)
        out["noise"] = g_eps.standard_normal(size=(T, E), dtype=np.float32)
    else:
        out["w_noise"] = None
        out["noise"] = None
    if cfg.bias == "hot8":
        b = np.zeros(E, dtype=np.float32)
        b[: min(8, E)] = 2.0
        out["gate_bias"] = b
    elif cfg.bias == "zipf":
        logit_std = float(np.sqrt(d * cfg.x_std**2 * cfg.wg_std**2))
        out["gate_bias"] = zipf_gate_bias(E, 1.2, logit_std).copy()
    else:
        out["gate_bias"] = None
    if with_weights:
        out["w1"] = _expert_stack(ss[4], E, (d, f), cfg.w1_std, cfg.dtype)
        out["w2"] = _expert_stack(ss[5], E, (f, d), cfg.w2_std, cfg.dtype)
    return out
