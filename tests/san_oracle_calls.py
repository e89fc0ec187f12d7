"""Calls every function of the oracle's C library on small inputs (ragged,
capacity-bound, noisy, fp32 and bf16, both drop orders, the backward, the
two-level gate and the noise stream). Run as a script by test_sanitizers.py
with an AddressSanitizer / UndefinedBehaviorSanitizer build of the library
loaded through MOE_ORACLE_LIB; prints one line per step and "OK" at the end.
"""

from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
from synthetic import CONFIGS, HIER_CONFIGS, hier_scaled, make_hier_inputs, make_inputs, scaled  # noqa: E402


def step(name):
    print(name, flush=True)


def main():
    print(f"library {oracle._lib()._name}", flush=True)
    step("element-wise functions")
    z = np.linspace(-30, 30, 4097).astype(np.float32)
    oracle.softplus(z)
    oracle.exp_nonpos(-np.abs(z))
    oracle.log1p_unit(np.linspace(0, 1, 1001).astype(np.float32))
    oracle.capacity(1000, 7, 2, 1.25)

    shapes = [
        ("tiny_fp32", dict(T=37), -1, False),
        ("switch_top1", dict(T=203, E=8, d_model=40, d_ff=24), 5, False),
        ("noisy_top4", dict(T=150, E=12, k=3, d_model=24, d_ff=40), -1, False),
        ("gshard_top2", dict(T=120, E=6, d_model=32, d_ff=16), 9, True),
        ("dropless_top1", dict(T=99, E=5, d_model=16, d_ff=24), -1, False),
    ]
    for name, over, cap, slot_major in shapes:
        cfg = scaled(CONFIGS[name], **over)
        inp = make_inputs(cfg)
        spec = oracle.LayerSpec.of(cfg, capacity=cap, slot_major=slot_major)
        step(f"forward {cfg.name} C={cap} slot_major={slot_major}")
        out = oracle.forward(spec, inp)
        assert np.isfinite(out["y"]).all()
        step(f"backward {cfg.name}")
        rng = np.random.default_rng(1)
        dy = rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
        b = oracle.backward(spec, inp, dy, (0.01, 0.01, 0.01))
        assert all(np.isfinite(v).all() for v in b.values() if isinstance(v, np.ndarray))

    for over in ({}, dict(T=70, groups=3, experts_per_group=5, k_group=2, k=2)):
        cfg = hier_scaled(HIER_CONFIGS["hier_tiny"], **over) if over else HIER_CONFIGS["hier_tiny"]
        step(f"forward_hier {cfg.name}")
        out = oracle.forward_hier(oracle.HierSpec.of(cfg, capacity=4), make_hier_inputs(cfg))
        assert np.isfinite(out["y"]).all()

    step("noise")
    oracle.philox_words(5, 9, 13, row0=(1 << 32) - 4)
    oracle.normal_noise(5, 33, 17)
    w = np.random.default_rng(2).integers(0, 2**32, size=(1000, 2), dtype=np.uint64).astype(np.uint32)
    oracle.normal_from_words(w)
    print("OK", flush=True)


if __name__ == "__main__":
    main()
