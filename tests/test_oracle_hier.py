"""Pins for the oracle's hierarchical MoE (Shazeer et al. summary page,
"Schluesselbegriffe": a primary gating network routes each input to secondary
MoE groups; "moe paper models" table 2: k = 2 for the hierarchical models).

Independent routes: the degenerate shapes that reduce to the flat layer (one
group; one expert per group), a brute-force dense evaluation over all group
and expert subsets on tiny inputs, the gate sum, and the losses by plain loops.
"""

import itertools
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import erf, softmax

from synthetic import CONFIGS, HIER_CONFIGS, hier_scaled, make_hier_inputs


def _act(z, act):
    return np.maximum(z, 0.0) if act == "relu" else 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def _flat_spec(orc, cfg, E, k, dtype):
    return orc.LayerSpec(cfg.T, cfg.d_model, cfg.d_ff, E, k, dtype, cfg.act, True)


def test_one_group_is_the_flat_layer(orc):
    """a = 1, k_group = 1: the primary gate is softmax over one kept logit = 1
    exactly, so routing, gates and y are the flat layer's with the secondary gate."""
    cfg = hier_scaled(HIER_CONFIGS["hier_tiny"], groups=1, experts_per_group=6, k_group=1, k=3)
    inp = make_hier_inputs(cfg)
    spec = orc.HierSpec.of(cfg)
    h = orc.forward_hier(spec, inp)
    flat = dict(x=inp["x"], w_gate=inp["w_gate_s"], w_noise=inp["w_noise_s"], noise=inp["noise_s"], w1=inp["w1"],
                w2=inp["w2"])
    f = orc.forward(_flat_spec(orc, cfg, 6, 3, cfg.dtype), flat)
    assert np.array_equal(h["topk_idx"], f["topk_idx"])
    assert np.array_equal(h["topk_gate"], f["topk_gate"])
    assert np.allclose(h["y"], f["y"], rtol=1e-13, atol=1e-14)
    assert h["aux"][1] == pytest.approx(f["aux"][1], rel=1e-12)


def test_one_expert_per_group_is_the_flat_layer(orc):
    """b = 1, k = 1: each group's gate is 1 exactly, so the layer is the flat
    layer gated by the primary gate (its load loss included)."""
    cfg = hier_scaled(HIER_CONFIGS["hier_tiny"], groups=5, experts_per_group=1, k_group=2, k=1)
    inp = make_hier_inputs(cfg)
    h = orc.forward_hier(orc.HierSpec.of(cfg), inp)
    flat = dict(x=inp["x"], w_gate=inp["w_gate_p"], w_noise=inp["w_noise_p"], noise=inp["noise_p"], w1=inp["w1"],
                w2=inp["w2"])
    f = orc.forward(_flat_spec(orc, cfg, 5, 2, cfg.dtype), flat)
    assert np.array_equal(h["topk_idx"], f["topk_idx"])
    assert np.allclose(h["topk_gate"], f["topk_gate"], rtol=1e-15, atol=0)
    assert np.allclose(h["y"], f["y"], rtol=1e-13, atol=1e-14)
    assert h["aux"][0] == pytest.approx(f["aux"][1], rel=1e-12)  # primary importance = the flat importance
    assert h["aux"][2] == pytest.approx(f["aux"][2], rel=1e-12)  # primary load = the flat load


def _best_subset(vals, k):
    """Lexicographically smallest index set of k entries with the largest sum."""
    best = None
    for sub in itertools.combinations(range(len(vals)), k):
        s = sum(float(vals[i]) for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    return list(best[1])


@settings(max_examples=20, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(T=st.integers(1, 12), a=st.integers(1, 4), b=st.integers(1, 4), kpf=st.floats(0, 1), ksf=st.floats(0, 1),
       act=st.sampled_from(["relu", "gelu"]), seed=st.integers(0, 10_000))
def test_matches_brute_force_dense(orc, T, a, b, kpf, ksf, act, seed):
    kp = 1 + int(kpf * (a - 1))
    ks = 1 + int(ksf * (b - 1))
    if kp * ks > 8:
        ks = max(1, 8 // kp)
    cfg = hier_scaled(HIER_CONFIGS["hier_tiny"], T=T, groups=a, experts_per_group=b, k_group=kp, k=ks, d_model=8,
                      d_ff=16, act=act)
    inp = make_hier_inputs(cfg, seed=seed)
    h = orc.forward_hier(orc.HierSpec.of(cfg), inp)
    x = inp["x"].astype(np.float64)
    w1, w2 = inp["w1"].astype(np.float64), inp["w2"].astype(np.float64)
    Hp, Hs = h["Hp"], h["Hs"]  # the canonical logits (pinned in test_oracle_routing)
    y = np.zeros_like(x)
    for t in range(T):
        groups = _best_subset(Hp[t], kp)
        gp = softmax(Hp[t, groups].astype(np.float64))
        for gi, grp in zip(gp, groups):
            hs = Hs[t, grp * b:(grp + 1) * b]
            ex = _best_subset(hs, ks)
            gs = softmax(hs[ex].astype(np.float64))
            for gj, j in zip(gs, ex):
                e = grp * b + j
                y[t] += gi * gj * (_act(x[t] @ w1[e], act) @ w2[e])
    assert np.allclose(h["y"], y, rtol=1e-10, atol=1e-12)
    assert np.allclose(h["topk_gate"].sum(axis=1), 1.0, atol=1e-14)


def _cv2(v):
    mu = sum(v) / len(v)
    return 0.0 if len(v) <= 1 else sum((a - mu) ** 2 for a in v) / len(v) / mu ** 2


def test_losses_by_plain_loops(orc):
    cfg = hier_scaled(HIER_CONFIGS["hier_tiny"], T=40)
    inp = make_hier_inputs(cfg, seed=3)
    h = orc.route_hier(orc.HierSpec.of(cfg), inp)
    a, b, kp = cfg.groups, cfg.experts_per_group, cfg.k_group
    clean, sigma, Hp = orc.gate_logits(inp["x"], inp["w_gate_p"], None, inp["w_noise_p"], inp["noise_p"], cfg.dtype)
    imp_p, imp_c, load_p = [0.0] * a, [0.0] * cfg.E, [0.0] * a
    for t in range(cfg.T):
        hp = [float(v) for v in Hp[t]]
        ranked = sorted(range(a), key=lambda i: (-hp[i], i))
        kept = ranked[:kp]
        m = max(hp[i] for i in kept)
        z = sum(math.exp(hp[i] - m) for i in kept)
        for i in kept:
            imp_p[i] += math.exp(hp[i] - m) / z
        for i in range(a):
            others = sorted((hp[j] for j in range(a) if j != i), reverse=True)
            zz = (float(clean[t, i]) - others[kp - 1]) / float(sigma[t, i])
            load_p[i] += 0.5 * math.erfc(-zz / math.sqrt(2.0))
        for s_ in range(cfg.slots):
            imp_c[int(h["topk_idx"][t, s_])] += float(h["topk_gate"][t, s_])
    assert h["aux"] == pytest.approx([_cv2(imp_p), _cv2(imp_c), _cv2(load_p)], rel=1e-10)


def test_hier_workload_shapes():
    c = HIER_CONFIGS["hier_top2x2"]
    assert (c.groups * c.experts_per_group, c.k_group, c.k) == (256, 2, 2)
    # the same expert shape and expert count as the noisy top-k workload
    n = CONFIGS["noisy_top4"]
    assert (c.T, c.d_model, c.d_ff, c.E, c.slots) == (n.T, n.d_model, n.d_ff, n.E, n.k)
