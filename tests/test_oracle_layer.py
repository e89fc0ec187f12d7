"""Pins for the oracle's expert FFN, combine and the composed layer.

Layer equation y = sum_i G(x)_i E_i(x) with experts as feed-forward
sub-networks (Shazeer et al. summary page, "Methode" and abstract); the
Switch listing adds each expert's output back at its tokens.
"""

import itertools

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import erf, softmax

from synthetic import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, scaled


def _f(a, dtype):
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def _act(z, act):
    return np.maximum(z, 0.0) if act == "relu" else 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_a_dense_ffn(orc, act, dtype):
    """E=1, k=1: the gate is exp(0)/exp(0) = 1 exactly, so the layer is the
    dense FFN act(x W1) W2 (numpy matmul)."""
    cfg = scaled(CONFIGS["tiny_fp32"], T=77, E=1, k=1, d_model=32, d_ff=96)
    cfg = cfg.__class__(**{**cfg.__dict__, "dtype": dtype, "act": act})
    inp = make_inputs(cfg)
    out = orc.forward(orc.LayerSpec.of(cfg), inp)
    assert np.all(out["topk_gate"] == 1.0)
    x = _f(inp["x"], dtype)
    ref = _act(x @ _f(inp["w1"][0], dtype), act) @ _f(inp["w2"][0], dtype)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def _identity_weights(E, d, f, dtype):
    """W1 = [I | -I | 0], W2 = [I ; -I ; 0] for every expert: act(z) - act(-z) = z
    for ReLU and for the exact GELU, so each expert is the identity map."""
    w1 = np.zeros((E, d, f), np.float32)
    w2 = np.zeros((E, f, d), np.float32)
    eye = np.eye(d, dtype=np.float32)
    w1[:, :, :d] = eye
    w1[:, :, d:2 * d] = -eye
    w2[:, :d, :] = eye
    w2[:, d:2 * d, :] = -eye
    if dtype == "bf16":
        return f32_to_bf16_bits(w1), f32_to_bf16_bits(w2)
    return w1, w2


@pytest.mark.parametrize("name", ["tiny_fp32", "switch_top1", "noisy_top4", "gshard_top2"])
def test_identity_experts_scale_x_by_kept_gate_sum(orc, name):
    base = CONFIGS[name]
    T = base.T if base.T <= 2048 else 1500
    cfg = scaled(base, T=T)
    d, f, E = cfg.d_model, cfg.d_ff, cfg.E
    if name != "tiny_fp32":  # keep the CPU FFN cheap: real d, smaller f >= 2d
        cfg = scaled(cfg, d_ff=2 * d)
        f = 2 * d
    inp = make_inputs(cfg, with_weights=False)
    inp["w1"], inp["w2"] = _identity_weights(E, d, f, cfg.dtype)
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(T, size=min(T, 96), replace=False))
    # a capacity that binds, so some slots are dropped
    C = max(1, (T * cfg.k) // (2 * E)) if cfg.capacity_factor > 0 else -1
    out = orc.forward(orc.LayerSpec.of(cfg, capacity=C), inp, tokens=tokens)
    kept_sum = np.where(out["slot_dest"][tokens] >= 0, out["topk_gate"][tokens], 0.0).sum(1)
    ref = kept_sum[:, None] * _f(inp["x"], cfg.dtype)[tokens]
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    if C >= 0:
        assert (out["slot_dest"] < 0).any()


def _brute_force_layer(x, H, w1, w2, k, act, renormalize):
    """Dense evaluation: every expert on every token, then the gate that keeps
    the lexicographically smallest max-sum k-subset of H (softmax over it, or
    the raw full-softmax probabilities)."""
    T, E = H.shape
    ys = np.stack([_act(x @ w1[e], act) @ w2[e] for e in range(E)])  # [E, T, d]
    y = np.zeros_like(x)
    p = softmax(H.astype(np.float64), axis=1)
    for t in range(T):
        best = None
        for sub in itertools.combinations(range(E), k):
            s = sum(float(H[t, e]) for e in sub)
            if best is None or s > best[0]:
                best = (s, sub)
        sub = list(best[1])
        g = softmax(H[t, sub].astype(np.float64)) if renormalize else p[t, sub]
        for gi, e in zip(g, sub):
            y[t] += gi * ys[e, t]
    return y


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(
    T=st.integers(1, 24),
    d=st.sampled_from([8, 16]),
    f=st.sampled_from([8, 24]),
    E=st.integers(1, 6),
    kfrac=st.floats(0.0, 1.0),
    act=st.sampled_from(["relu", "gelu"]),
    renorm=st.booleans(),
    zero_gate=st.booleans(),
    seed=st.integers(0, 10_000),
)
def test_layer_matches_brute_force_dense(orc, T, d, f, E, kfrac, act, renorm, zero_gate, seed):
    k = 1 + int(kfrac * (min(E, 3) - 1))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (np.round(rng.standard_normal((d, E)) * 4) / 8).astype(np.float32)  # coarse: ties happen
    if zero_gate:
        wg[:] = 0.0
    w1 = (rng.standard_normal((E, d, f)) / np.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, f, d)) / np.sqrt(f)).astype(np.float32)
    inp = dict(x=x, w_gate=wg, w1=w1, w2=w2)
    spec = orc.LayerSpec(T, d, f, E, k, "f32", act, renorm)
    out = orc.forward(spec, inp)
    ref = _brute_force_layer(x.astype(np.float64), out["H"], w1.astype(np.float64), w2.astype(np.float64), k,
                             act, renorm)
    assert np.allclose(out["y"], ref, rtol=1e-10, atol=1e-10)


def test_combine_drops_and_all_dropped_rows(orc):
    T, E, k, d = 40, 3, 2, 8
    rng = np.random.default_rng(3)
    H = rng.standard_normal((T, E)).astype(np.float32)
    H[:, 0] += 3.0
    idx = orc.topk_order(H, k)
    disp = orc.dispatch(idx, E, 5)
    g, _ = orc.gates(H, idx, True)
    yp = rng.standard_normal((max(disp["R"], 1), d))
    y = orc.combine(np.arange(T), disp["slot_dest"], g, yp)
    for t in range(T):
        want = np.zeros(d)
        for s in range(k):
            sl = disp["slot_dest"][t, s]
            if sl >= 0:
                want += g[t, s] * yp[sl]
        assert np.allclose(y[t], want, rtol=1e-14, atol=1e-14)
    dead = (disp["slot_dest"] < 0).all(1)
    assert dead.any() and np.all(y[dead] == 0.0)


def test_forward_outputs_are_consistent(orc):
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    out = orc.forward(orc.LayerSpec.of(cfg), inp)
    assert out["topk_idx"].shape == (cfg.T, cfg.k)
    assert np.array_equal(out["counts_routed"], np.bincount(out["topk_idx"].ravel(), minlength=cfg.E))
    assert out["R"] == cfg.T * cfg.k  # no capacity limit
    assert np.allclose(out["topk_gate"].sum(1), 1.0, atol=1e-14)
    assert np.isnan(out["aux"][2]) and np.isfinite(out["aux"][:2]).all()
