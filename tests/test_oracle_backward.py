"""Pins for the oracle's backward pass: central finite differences of the
oracle's own forward (the composed layer, pinned on its own elsewhere).

The loss is L = sum(dy * y) + w_switch * switch_aux + w_importance *
CV(Importance)^2 + w_load * CV(Load)^2 (Shazeer et al. summary page, "Methode"
and "Load-Balancing-Losses"; the "Switch Transformer" page's auxiliary loss).
Its gradient with respect to every parameter -- x, W_gate, gate_bias,
W_noise, W1, W2 -- must match (L(p + h) - L(p - h)) / 2h at sampled entries,
with the discrete choices (top-k sets, drops) unchanged by the step (checked;
the inputs are chosen with clear gaps). fp32 layers, so steps are continuous;
the gate logits are the forward's canonical fp32 values, whose rounding sets
the tolerance. A plausible slip in the backward -- a missing softmax-Jacobian
term, the load estimator's threshold gradient sent to the wrong expert, the
noise path's sigmoid, a dropped slot that still receives gradient -- moves
some entry far outside it.
"""

import numpy as np
import pytest

from synthetic import CONFIGS, make_inputs, scaled


def _loss(orc, spec, inp, dy, w):
    out = orc.forward(spec, inp)
    L = float((dy * out["y"]).sum()) + w[0] * out["aux"][0] + w[1] * out["aux"][1]
    if inp.get("w_noise") is not None:
        L += w[2] * out["aux"][2]
    return L, out["order"] if "order" in out else out["topk_idx"], out["slot_dest"]


def _check_param(orc, spec, inp, dy, w, name, grad, n_samples, rng, h=2e-3):
    base = inp[name]
    flat_idx = rng.choice(base.size, size=min(n_samples, base.size), replace=False)
    _, order0, slots0 = _loss(orc, spec, inp, dy, w)
    scale = np.abs(grad).max()
    checked = 0
    for fi in flat_idx:
        idx = np.unravel_index(fi, base.shape)
        vals = []
        steps = []
        for sgn in (+1, -1):
            q = dict(inp)
            arr = base.copy()
            arr[idx] = np.float32(arr[idx] + sgn * h)
            steps.append(float(arr[idx]))
            q[name] = arr
            L, order, slots = _loss(orc, spec, q, dy, w)
            if not (np.array_equal(order, order0) and np.array_equal(slots, slots0)):
                break  # a discrete choice moved: this entry is not differentiable here
            vals.append(L)
        if len(vals) < 2:
            continue
        fd = (vals[0] - vals[1]) / (steps[0] - steps[1])
        an = float(grad[idx])
        assert abs(fd - an) <= 2e-3 * scale + 5e-3 * abs(an), (name, idx, fd, an, scale)
        checked += 1
    assert checked >= max(1, n_samples // 2), f"{name}: only {checked} entries were differentiable"


CASES = [
    # noisy top-2 with all three losses (the load estimator's gradient included)
    dict(base="noisy_top4", T=24, E=6, k=2, d_model=12, d_ff=24, act="gelu", w=(0.3, 0.7, 0.9)),
    # noisy top-3 of 4, renormalised, ReLU experts (a smaller step: fewer hidden units cross the kink)
    dict(base="noisy_top4", T=20, E=4, k=3, d_model=8, d_ff=16, act="relu", w=(0.0, 0.5, 1.3), h=2e-4),
    # Switch-style raw top-1 gate with a binding capacity (dropped tokens get no expert gradient)
    dict(base="switch_top1", T=30, E=5, k=1, d_model=12, d_ff=24, act="gelu", w=(0.8, 0.4, 0.0), capacity=5),
    # top-2 renormalised with capacity, first-choice priority
    dict(base="gshard_top2", T=28, E=5, k=2, d_model=8, d_ff=16, act="gelu", w=(0.5, 0.5, 0.0), capacity=8,
         slot_major=True),
    # a single expert: the dense FFN backward
    dict(base="tiny_fp32", T=16, E=1, k=1, d_model=8, d_ff=16, act="gelu", w=(0.0, 0.0, 0.0)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c['base']}-E{c['E']}k{c['k']}" for c in CASES])
def test_backward_matches_finite_differences(orc, case):
    c = dict(case)
    base = CONFIGS[c.pop("base")]
    w = c.pop("w")
    cap = c.pop("capacity", -1)
    slot_major = c.pop("slot_major", False)
    act = c.pop("act")
    h = c.pop("h", 2e-3)
    cfg = scaled(base, **c)
    cfg = cfg.__class__(**{**cfg.__dict__, "dtype": "f32", "act": act})
    inp = make_inputs(cfg)
    if cfg.bias != "none" or base.name == "switch_top1":
        inp["gate_bias"] = np.linspace(-0.3, 0.3, cfg.E).astype(np.float32)
    spec = orc.LayerSpec.of(cfg, capacity=cap, slot_major=slot_major)
    rng = np.random.default_rng(11)
    dy = rng.standard_normal((cfg.T, cfg.d_model))
    b = orc.backward(spec, inp, dy, w)
    if cap >= 0:
        assert (b["disp"]["slot_dest"] < 0).any(), "the capacity should drop something"
    _check_param(orc, spec, inp, dy, w, "x", b["dx"], 12, rng, h)
    _check_param(orc, spec, inp, dy, w, "w_gate", b["dw_gate"], 10, rng, h)
    _check_param(orc, spec, inp, dy, w, "w1", b["dw1"], 10, rng, h)
    _check_param(orc, spec, inp, dy, w, "w2", b["dw2"], 10, rng, h)
    if inp.get("gate_bias") is not None:
        _check_param(orc, spec, inp, dy, w, "gate_bias", b["dgate_bias"], cfg.E, rng, h)
    if inp.get("w_noise") is not None:
        _check_param(orc, spec, inp, dy, w, "w_noise", b["dw_noise"], 10, rng, h)


def test_dropped_assignments_get_no_expert_gradient(orc):
    """A token whose only slot is dropped contributes nothing to y, so dy on it
    reaches neither the experts nor (without losses) the gate."""
    cfg = scaled(CONFIGS["switch_top1"], T=40, E=4, d_model=8, d_ff=16)
    cfg = cfg.__class__(**{**cfg.__dict__, "dtype": "f32"})
    inp = make_inputs(cfg)
    spec = orc.LayerSpec.of(cfg, capacity=3)
    dead = None
    dy = np.zeros((cfg.T, cfg.d_model))
    b0 = orc.backward(spec, inp, dy)
    dead = np.flatnonzero(b0["disp"]["slot_dest"][:, 0] < 0)
    assert dead.size
    dy[dead] = 1.0
    b = orc.backward(spec, inp, dy)
    assert np.all(b["dw1"] == 0) and np.all(b["dw2"] == 0) and np.all(b["dx"] == 0)
    assert np.all(b["dw_gate"] == 0)


def test_subset_backward_equals_full_rows(orc):
    """The token / expert restriction used at full sizes returns exactly the
    full backward's rows (same per-token arithmetic, batch statistics shared)."""
    cfg = scaled(CONFIGS["noisy_top4"], T=60, E=8, k=2, d_model=16, d_ff=32)
    inp = make_inputs(cfg)
    spec = orc.LayerSpec.of(cfg, capacity=12)
    dy = np.random.default_rng(4).standard_normal((cfg.T, cfg.d_model))
    w = (0.2, 0.3, 0.4)
    full = orc.backward(spec, inp, dy, w)
    toks = np.array([0, 5, 17, 59])
    exps = np.array([1, 6])
    sub = orc.backward(spec, inp, dy, w, tokens=toks, experts=exps)
    assert np.allclose(sub["dx"], full["dx"][toks], rtol=1e-12, atol=1e-14)
    assert np.allclose(sub["dclean"], full["dclean"][toks], rtol=1e-12, atol=1e-14)
    assert np.allclose(sub["du"], full["du"][toks], rtol=1e-12, atol=1e-14)
    for e in exps:
        assert np.allclose(sub["dw1"][e], full["dw1"][e], rtol=1e-12, atol=1e-14)
        assert np.allclose(sub["dw2"][e], full["dw2"][e], rtol=1e-12, atol=1e-14)
