"""Pins for how ``oracle.route()`` assembles the balancing losses.

The loss terms themselves are pinned in ``test_oracle_routing.py``; here the
composed ``route()`` call is checked end to end against what the pages define,
recomputed independently:

* Shazeer et al. summary page, "Load-Balancing-Losses": Importance(X) is the
  batch sum of the gate vector G(x); the load of expert i is the batch sum of
  P(x, i) = Phi((clean_i - kth_excluding(H(x), k, i)) / Softplus((x W_noise)_i)),
  the probability that expert i stays in the top k when only its own noise is
  drawn again; each loss is CV(.)^2 of its vector.
* "Switch Transformer" page: an auxiliary load-balancing loss (read as
  E * sum_e f_e * P_e, f_e the routed fraction, P_e the mean full-softmax
  probability).

Independent routes: closed forms on degenerate gates, plain-Python loops over
tokens and experts (sorting for kth_excluding, math.erfc for Phi, math.exp for
the softmaxes), and a Monte Carlo estimate of the load made by re-drawing one
expert's noise column and running the whole ``route()`` call again.
"""

import math

import numpy as np
import pytest
from scipy.special import softmax

from synthetic import f32_to_bf16_bits


def _spec(orc, T, d, E, k, renormalize, dtype="f32"):
    return orc.LayerSpec(T, d, 4 * d, E, k, dtype, "relu", renormalize)


def _inputs(T, d, E, seed, noisy, bias=None):
    rng = np.random.default_rng(seed)
    inp = dict(x=rng.standard_normal((T, d)).astype(np.float32),
               w_gate=(rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32))
    if noisy:
        inp["w_noise"] = (rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
        inp["noise"] = rng.standard_normal((T, E)).astype(np.float32)
    if bias is not None:
        inp["gate_bias"] = np.asarray(bias, np.float32)
    return inp


@pytest.mark.parametrize("k,renorm", [(1, False), (2, True), (3, True), (2, False)])
def test_zero_gate_closed_forms(orc, k, renorm):
    """W_g = 0: every logit ties, so every token takes experts 0..k-1 (lower
    index first). P is uniform (1/E), so switch_aux = 1 for any f. Importance
    is (T*g_0, ..., T*g_{k-1}, 0, ...) with equal gates, whose population
    CV^2 is E/k - 1 in closed form."""
    T, d, E = 64, 16, 8
    inp = _inputs(T, d, E, 1, noisy=False)
    inp["w_gate"][:] = 0.0
    r = orc.route(_spec(orc, T, d, E, k, renorm), inp)
    assert np.all(r["topk_idx"] == np.arange(k))
    assert r["aux"][0] == pytest.approx(1.0, abs=1e-14)
    assert r["aux"][1] == pytest.approx(E / k - 1.0, rel=1e-12)
    assert np.isnan(r["aux"][2])


def test_all_tokens_on_one_expert(orc):
    """A bias that sends every token to expert j: f is one-hot at j, so
    switch_aux = E * P_j (P_j = batch mean of softmax(H)_j, here from scipy),
    and importance is one-hot, whose CV^2 is E - 1."""
    T, d, E, j = 96, 16, 6, 4
    bias = np.zeros(E, np.float32)
    bias[j] = 30.0
    inp = _inputs(T, d, E, 2, noisy=False, bias=bias)
    r = orc.route(_spec(orc, T, d, E, 1, False), inp)
    assert np.all(r["topk_idx"][:, 0] == j)
    P_j = softmax(r["H"].astype(np.float64), axis=1)[:, j].mean()
    assert r["aux"][0] == pytest.approx(E * P_j, rel=1e-12)
    assert r["aux"][1] == pytest.approx(E - 1.0, rel=1e-12)


def _cv2(v):
    n = len(v)
    if n <= 1:
        return 0.0
    mean = sum(v) / n
    var = sum((a - mean) ** 2 for a in v) / n
    return var / mean ** 2


def _losses_by_loops(H, clean, sigma, k, renorm):
    """The three losses from their definitions, one token and expert at a time."""
    T, E = H.shape
    counts = [0] * E
    prob_sum = [0.0] * E
    importance = [0.0] * E
    load = [0.0] * E
    for t in range(T):
        h = [float(v) for v in H[t]]
        # top-k: H descending, the lower expert index first on ties
        ranked = sorted(range(E), key=lambda e: (-h[e], e))
        kept = ranked[:k]
        m = max(h)
        z = sum(math.exp(v - m) for v in h)
        p = [math.exp(v - m) / z for v in h]
        if renorm:
            zk = sum(math.exp(h[e] - m) for e in kept)
            g = [math.exp(h[e] - m) / zk for e in kept]
        else:
            g = [p[e] for e in kept]
        for e, ge in zip(kept, g):
            counts[e] += 1
            importance[e] += ge
        for e in range(E):
            prob_sum[e] += p[e]
        if sigma is not None:
            for e in range(E):
                others = sorted((h[j] for j in range(E) if j != e), reverse=True)
                if k > len(others):
                    load[e] += 1.0  # fewer than k rivals: always kept
                    continue
                kth = others[k - 1]  # kth_excluding(H, k, e)
                zval = (float(clean[t, e]) - kth) / float(sigma[t, e])
                load[e] += 0.5 * math.erfc(-zval / math.sqrt(2.0))
    switch = E * sum((counts[e] / (T * k)) * (prob_sum[e] / T) for e in range(E))
    return switch, _cv2(importance), (_cv2(load) if sigma is not None else float("nan")), load, importance


@pytest.mark.parametrize("noisy,k,renorm,E", [(True, 2, True, 6), (True, 1, True, 5), (True, 4, True, 4),
                                              (False, 1, False, 7), (False, 2, True, 5)])
def test_losses_match_plain_loops(orc, noisy, k, renorm, E):
    T, d = 50, 12
    inp = _inputs(T, d, E, 10 + E + k, noisy=noisy, bias=np.linspace(-0.5, 0.5, E))
    r = orc.route(_spec(orc, T, d, E, k, renorm), inp)
    # logits from the (separately pinned) gate itself, not from route()'s own dict
    clean, sigma, H = orc.gate_logits(inp["x"], inp["w_gate"], inp["gate_bias"], inp.get("w_noise"),
                                      inp.get("noise"), "f32")
    sw, cvi, cvl, load, imp = _losses_by_loops(H, clean, sigma, k, renorm)
    assert r["aux"][0] == pytest.approx(sw, rel=1e-12)
    assert r["aux"][1] == pytest.approx(cvi, rel=1e-10, abs=1e-14)
    assert np.allclose(r["importance"], imp, rtol=1e-12)
    if noisy:
        assert r["aux"][2] == pytest.approx(cvl, rel=1e-10, abs=1e-14)
        assert np.allclose(r["load"], load, rtol=1e-12)
    else:
        assert np.isnan(r["aux"][2])


def test_load_matches_monte_carlo_through_route(orc):
    """Load_e = sum_t P(t, e), P(t, e) the probability that e is in token t's top
    k when only its noise eps[t, e] is drawn again. Estimate it by re-drawing the
    whole column eps[:, e] M times (tokens are independent, so one column redraw
    samples every token's P(t, e) at once) and counting top-k membership in the
    topk_idx that route() itself returns; all M copies go through one route()
    call as a stacked batch."""
    T, d, E, k, M = 24, 12, 6, 2, 3000
    inp = _inputs(T, d, E, 7, noisy=True, bias=np.array([0.4, 0.0, -0.2, 0.3, -0.4, 0.1]))
    r = orc.route(_spec(orc, T, d, E, k, True), inp)
    rng = np.random.default_rng(123)
    big = dict(x=np.tile(inp["x"], (M, 1)), w_gate=inp["w_gate"], w_noise=inp["w_noise"],
               gate_bias=inp["gate_bias"])
    for e in range(E):
        noise = np.tile(inp["noise"], (M, 1))
        noise[:, e] = rng.standard_normal(M * T).astype(np.float32)
        big["noise"] = noise
        rb = orc.route(_spec(orc, M * T, d, E, k, True), big)
        hits = (rb["topk_idx"] == e).any(axis=1).reshape(M, T).mean(axis=0)  # P(t, e) estimates
        est = hits.sum()
        sd = math.sqrt(max((hits * (1 - hits)).sum(), 1e-12) / M)
        assert abs(est - r["load"][e]) <= 4.5 * sd + 1e-9, (e, est, r["load"][e], sd)


def test_bf16_route_losses_match_plain_loops(orc):
    """The same composition on a bf16 layer with a hot-expert bias (the noisy
    workload's kind of skew)."""
    T, d, E, k = 40, 16, 8, 2
    rng = np.random.default_rng(5)
    inp = dict(x=f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)),
               w_gate=f32_to_bf16_bits((rng.standard_normal((d, E)) / 4).astype(np.float32)),
               w_noise=f32_to_bf16_bits((rng.standard_normal((d, E)) / 4).astype(np.float32)),
               noise=rng.standard_normal((T, E)).astype(np.float32),
               gate_bias=np.where(np.arange(E) < 2, 2.0, 0.0).astype(np.float32))
    r = orc.route(_spec(orc, T, d, E, k, True, "bf16"), inp)
    clean, sigma, H = orc.gate_logits(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w_noise"], inp["noise"],
                                      "bf16")
    sw, cvi, cvl, _, _ = _losses_by_loops(H, clean, sigma, k, True)
    assert r["aux"] == pytest.approx([sw, cvi, cvl], rel=1e-10)
