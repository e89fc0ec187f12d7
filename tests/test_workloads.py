"""The workload table against the shapes the page tables fix, and the seeded
generators' recipe (reproducibility, distributions)."""

import os

import numpy as np

from synthetic import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")


def _facts():
    out = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            key, val, _ = line.split(" ", 2)
            out[key] = val
    return out


def test_workloads_follow_page_tables():
    f = _facts()
    sw, nz, gs, dl = (CONFIGS[n] for n in ("switch_top1", "noisy_top4", "gshard_top2", "dropless_top1"))
    assert sw.E == int(f["switch.E"]) and sw.d_model == int(f["switch.ffn"]) and sw.k == int(f["switch.k"])
    assert sw.capacity_factor == float(f["stmoe.capacity_factor"])
    assert nz.E == int(f["shazeer.E"]) and nz.k == int(f["shazeer.k"])
    assert sorted((nz.d_ff, nz.d_model)) == sorted(int(v) for v in f["shazeer.expert_dims"].split("x"))
    assert gs.k == int(f["gshard.k"]) and gs.E == int(f["fastermoe.E"])
    assert (gs.d_model, gs.d_ff) == tuple(int(v) for v in f["fastermoe.ffn"].split("/")[0::2])
    assert gs.capacity_factor == float(f["glam.capacity_factor"])
    assert dl.E == int(f["megablocks.E"]) and dl.k == int(f["megablocks.k"])


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38, 1e-30], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    assert got[0] == 1.0
    assert got[1] == 1.0  # exact tie -> even (1.0)
    assert got[2] == np.float32(1.0 + 4 * 2**-8)  # tie -> even (up)
    assert got[3] == 1.0
    assert got[4] == -2.5
    assert np.all(np.abs(got - vals) <= np.abs(vals) * 2**-8 + 1e-45)


def test_generators_are_seeded_and_shaped():
    cfg = scaled(CONFIGS["noisy_top4"], T=64)
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (64, 512) and a["x"].dtype == np.uint16
    assert a["noise"].shape == (64, 256) and a["noise"].dtype == np.float32
    assert a["w1"].shape == (256, 512, 1024) and a["w2"].shape == (256, 1024, 512)
    assert np.array_equal(a["gate_bias"][:8], np.full(8, 2.0, np.float32)) and not a["gate_bias"][8:].any()
    c = make_inputs(cfg, seed=1, with_weights=False)
    assert not np.array_equal(a["x"], c["x"])
    # x ~ N(0,1) survives bf16 rounding
    xf = bf16_bits_to_f32(a["x"])
    assert abs(xf.mean()) < 0.02 and abs(xf.std() - 1.0) < 0.02


def test_zipf_bias_shares():
    """The calibrated bias gives top-1 shares close to Zipf(1.2) under
    independent N(0,1) logit noise (Monte Carlo over fresh draws)."""
    cfg = CONFIGS["dropless_top1"]
    b = make_inputs(scaled(cfg, T=8), with_weights=False)["gate_bias"]
    rng = np.random.default_rng(0)
    z = rng.standard_normal((200_000, cfg.E)) + b
    share = np.bincount(z.argmax(1), minlength=cfg.E) / z.shape[0]
    target = np.arange(1, cfg.E + 1) ** -1.2
    target /= target.sum()
    assert 0.5 * np.abs(share - target).sum() < 0.01
