"""Hierarchical MoE workloads (two-level gating) and their seeded inputs.

The Shazeer et al. summary page ("Schluesselbegriffe") names a hierarchical
MoE: a primary gating network routes each input to secondary MoE groups; the
"moe paper models" page, table 2, gives k = 2 for the hierarchical (MoE-H)
models. A layer here has ``groups`` secondary MoEs of ``experts_per_group``
experts each; the primary gate keeps ``k_group`` groups and each kept group's
gate keeps ``k`` of its experts, so a token has k_group * k expert slots.

Like ``generate.py`` this module holds shapes, distributions and the random
number recipe only -- no arithmetic of the layer. Streams:
``SeedSequence(seed).spawn(8)`` in the order x, W_gate_primary,
W_noise_primary, noise_primary, W_gate_secondary, W_noise_secondary,
noise_secondary, then the expert weights (W1 and W2 from two children of the
last stream).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

from .generate import _expert_stack, _normal


@dataclass(frozen=True)
class HierConfig:
    name: str
    T: int
    d_model: int
    d_ff: int
    groups: int
    experts_per_group: int
    k_group: int
    k: int
    dtype: str
    act: str
    noisy: bool
    capacity_factor: float = 0.0
    description: str = ""

    @property
    def E(self) -> int:
        return self.groups * self.experts_per_group

    @property
    def slots(self) -> int:
        return self.k_group * self.k


HIER_CONFIGS = {
    c.name: c
    for c in [
        # 16 groups x 16 experts (the expert shape of the noisy top-k workload), k = 2 at both
        # levels, noisy gates at both levels
        HierConfig("hier_top2x2", 8192, 512, 1024, 16, 16, 2, 2, "bf16", "relu", True,
                   description="T=8192 d=512 f=1024, 16 groups x 16 experts, top-2 groups x top-2 experts, "
                               "noisy gates, ReLU bf16"),
        HierConfig("hier_tiny", 128, 32, 64, 4, 3, 2, 2, "f32", "gelu", True,
                   description="T=128 d=32 f=64, 4 groups x 3 experts, top-2 x top-2, noisy, GELU fp32"),
    ]
}


def hier_scaled(cfg: HierConfig, **changes) -> HierConfig:
    new = replace(cfg, **changes)
    return replace(new, name=f"{cfg.name}[T={new.T},d={new.d_model},f={new.d_ff},a={new.groups},"
                             f"b={new.experts_per_group},kp={new.k_group},k={new.k}]")


def make_hier_inputs(cfg: HierConfig, seed: int = 0) -> dict:
    """x [T,d]; w_gate_p [d,groups] and w_gate_s [d,E] (E = groups * experts_per_group;
    column g*b + j is expert j of group g); with noisy gates also w_noise_p,
    w_noise_s and standard-normal noise_p [T,groups], noise_s [T,E] (fp32);
    w1 [E,d,f], w2 [E,f,d]. Gate weights N(0, 1/d), experts N(0, 1/fan_in), x N(0, 1)."""
    T, d, f, a, E = cfg.T, cfg.d_model, cfg.d_ff, cfg.groups, cfg.E
    ss = np.random.SeedSequence(seed).spawn(8)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss[:7]]
    std = math.sqrt(1.0 / d)
    out = {
        "x": _normal(g[0], (T, d), 1.0, cfg.dtype),
        "w_gate_p": _normal(g[1], (d, a), std, cfg.dtype),
        "w_gate_s": _normal(g[4], (d, E), std, cfg.dtype),
        "w_noise_p": None, "noise_p": None, "w_noise_s": None, "noise_s": None,
    }
    if cfg.noisy:
        out["w_noise_p"] = _normal(g[2], (d, a), std, cfg.dtype)
        out["noise_p"] = g[3].standard_normal(size=(T, a), dtype=np.float32)
        out["w_noise_s"] = _normal(g[5], (d, E), std, cfg.dtype)
        out["noise_s"] = g[6].standard_normal(size=(T, E), dtype=np.float32)
    w1s, w2s = ss[7].spawn(2)
    out["w1"] = _expert_stack(w1s, E, (d, f), math.sqrt(1.0 / d), cfg.dtype)
    out["w2"] = _expert_stack(w2s, E, (f, d), math.sqrt(1.0 / f), cfg.dtype)
    return out
