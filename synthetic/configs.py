"""The five layer workloads and their input distributions.

Shapes follow the MoE layers listed on the pages:

* tiny_fp32      -- a small fp32 layer the oracle evaluates in well under a second.
* switch_top1    -- Switch Transformer entry (dictionary page "Switch Transformer":
                    top-1 routing) with the Switch shape from the "moe paper models"
                    table 1 (768 FFN size, 128 experts) and the ST-MoE capacity
                    factor 1.25 from table 2.
* noisy_top4     -- Shazeer et al. summary page, "Methode": noisy top-k gating;
                    expert shape 1024x512 and 256 experts from table 1 of
                    "moe paper models", k=4 from its table 2.
* gshard_top2    -- top-2 routing with capacity factor 2 (GShard / FasterMoE rows
                    of "moe paper models" tables 1 and 2; 1024/4096 FFN, 64 experts).
* dropless_top1  -- MegaBlocks row (64 experts, top-1) of "moe paper models",
                    no capacity limit, Zipf-skewed segment sizes.

``N(0, v)`` in the workload descriptions is read as variance ``v``; the
``*_std`` fields below are the corresponding standard deviations.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    dtype: str  # "f32" or "bf16": storage type of x, W_gate, W_noise, W1, W2, Xp, Yp, y
    act: str  # "relu" or "gelu" (exact erf form)
    renormalize: bool  # True: softmax over the k kept logits; False: raw full-softmax probability
    capacity_factor: float  # <= 0 means no capacity limit
    noisy: bool  # noisy top-k gating (W_noise and a standard-normal noise tensor)
    x_std: float
    wg_std: float
    wn_std: float
    w1_std: float
    w2_std: float
    bias: str  # "none", "hot8" (+2 on experts 0..7) or "zipf" (Zipf(s=1.2) segment sizes)
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.T


def _cfg(**kw) -> MoEConfig:
    return MoEConfig(**kw)


CONFIGS: dict[str, MoEConfig] = {
    c.name: c
    for c in [
        _cfg(
            name="tiny_fp32", T=256, d_model=64, d_ff=256, E=4, k=2, dtype="f32", act="relu",
            renormalize=True, capacity_factor=0.0, noisy=False,
            x_std=1.0, wg_std=math.sqrt(1 / 64), wn_std=0.0,
            w1_std=math.sqrt(1 / 64), w2_std=math.sqrt(1 / 256), bias="none",
            description="T=256 d=64 f=256 E=4 top-2 renormalised, no capacity, ReLU, fp32",
        ),
        _cfg(
            name="switch_top1", T=16384, d_model=768, d_ff=3072, E=128, k=1, dtype="bf16",
            act="gelu", renormalize=False, capacity_factor=1.25, noisy=False,
            x_std=1.0, wg_std=math.sqrt(1e-2), wn_std=0.0,
            w1_std=math.sqrt(1 / 768), w2_std=math.sqrt(1 / 3072), bias="none",
            description="T=16384 (8x2048) d=768 f=3072 E=128 top-1 cf=1.25 GELU bf16",
        ),
        _cfg(
            name="noisy_top4", T=8192, d_model=512, d_ff=1024, E=256, k=4, dtype="bf16",
            act="relu", renormalize=True, capacity_factor=0.0, noisy=True,
            x_std=1.0, wg_std=math.sqrt(1 / 512), wn_std=math.sqrt(1 / 512),
            w1_std=math.sqrt(1 / 512), w2_std=math.sqrt(1 / 1024), bias="hot8",
            description="T=8192 d=512 f=1024 E=256 noisy top-4, +2 on 8 hot experts, ReLU bf16",
        ),
        _cfg(
            name="gshard_top2", T=32768, d_model=1024, d_ff=4096, E=64, k=2, dtype="bf16",
            act="gelu", renormalize=True, capacity_factor=2.0, noisy=False,
            x_std=1.0, wg_std=math.sqrt(1e-3), wn_std=0.0,
            w1_std=math.sqrt(1 / 1024), w2_std=math.sqrt(1 / 4096), bias="none",
            description="T=32768 (16x2048) d=1024 f=4096 E=64 top-2 cf=2.0 GELU bf16",
        ),
        _cfg(
            name="dropless_top1", T=65536, d_model=2048, d_ff=8192, E=64, k=1, dtype="bf16",
            act="gelu", renormalize=False, capacity_factor=0.0, noisy=False,
            x_std=1.0, wg_std=math.sqrt(1 / 2048), wn_std=0.0,
            w1_std=math.sqrt(1 / 2048), w2_std=math.sqrt(1 / 8192), bias="zipf",
            description="T=65536 d=2048 f=8192 E=64 dropless top-1, Zipf(1.2) segments, GELU bf16",
        ),
    ]
}

CONFIG_ORDER = ["tiny_fp32", "switch_top1", "noisy_top4", "gshard_top2", "dropless_top1"]


def get_config(name: str) -> MoEConfig:
    if name not in CONFIGS:
        raise KeyError(f"unknown MoE workload {name!r}; known: {', '.join(CONFIG_ORDER)}")
    return CONFIGS[name]


def scaled(cfg: MoEConfig, **changes) -> MoEConfig:
    """A copy of ``cfg`` with some shape fields replaced (same distributions).

    Standard deviations that are defined as ``1/fan_in`` variances follow the new
    fan-in so that activations keep unit scale.
    """
    new = replace(cfg, **changes)
    d, f = new.d_model, new.d_ff
    upd = {}
    if "d_model" in changes:
        upd["w1_std"] = math.sqrt(1 / d)
        if cfg.wg_std == math.sqrt(1 / cfg.d_model):
            upd["wg_std"] = math.sqrt(1 / d)
        if cfg.noisy:
            upd["wn_std"] = math.sqrt(1 / d)
    if "d_ff" in changes:
        upd["w2_std"] = math.sqrt(1 / f)
    if upd:
        new = replace(new, **upd)
    return replace(new, name=f"{cfg.name}[T={new.T},d={d},f={f},E={new.E},k={new.k}]")
