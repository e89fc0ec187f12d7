"""Pins for the oracle's routing: gate logits, top-k, gate values, capacity,
dispatch and the balancing losses.

Method sources: Shazeer et al. summary page ("Methode": layer equation, Noisy
Top-K Gating, Load-Balancing-Losses), the "Switch Transformer" page (top-1
routing; softmax over all experts; gate = mask * weights) and table 2 of the
"moe paper models" page (capacity factors). Each test ties the oracle to
something other than itself: exact rational arithmetic, numpy/scipy library
routines, brute force, closed forms and invariants.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr, softmax

from fp32exact import add_f32, fma_f32
from synthetic import CONFIGS, f32_to_bf16_bits, make_inputs, scaled


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, np.float32))


def _widen(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# gate logits
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logits_equal_exact_sequential_fma_chain(orc, dtype):
    """Bit-exact against an independent emulation of the canonical order:
    acc = +0; acc = fma(x_j, w_je, acc) for j ascending; then + bias."""
    rng = np.random.default_rng(5)
    T, d, E = 3, 24, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((d, E)) * 0.3).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    if dtype == "bf16":
        x, w = _bf16(x), _bf16(w)
        xf, wf = _widen(x), _widen(w)
    else:
        xf, wf = x, w
    clean, _, H = orc.gate_logits(x, w, b, dtype=dtype)
    for t in range(T):
        for e in range(E):
            acc = Fraction(0)
            for j in range(d):
                acc = fma_f32(float(xf[t, j]), float(wf[j, e]), acc)
            ref = add_f32(acc, float(b[e]))
            assert Fraction(float(clean[t, e])) == ref
    assert np.array_equal(clean, H)


def test_logits_one_hot_rows_are_exact(orc):
    rng = np.random.default_rng(6)
    d, E = 32, 7
    w = _bf16(rng.standard_normal((d, E)))
    x = np.zeros((d, d), np.float32)
    x[np.arange(d), np.arange(d)] = 1.0
    clean, _, _ = orc.gate_logits(_bf16(x), w, dtype="bf16")
    assert np.array_equal(clean, _widen(w))


def test_logits_within_rounding_bound_of_exact_dot(orc):
    """|fl(dot) - dot| <= d * 2^-24 * sum |x_j w_je| (any fp32 summation order)."""
    cfg = scaled(CONFIGS["switch_top1"], T=64)
    inp = make_inputs(cfg, with_weights=False)
    clean, _, _ = orc.gate_logits(inp["x"], inp["w_gate"], dtype="bf16")
    xf = _widen(inp["x"]).astype(np.float64)
    wf = _widen(inp["w_gate"]).astype(np.float64)
    exact = xf @ wf  # products of bf16 values are exact in fp64 and d*2^-53 is negligible here
    bound = cfg.d_model * 2.0**-24 * (np.abs(xf) @ np.abs(wf))
    assert np.all(np.abs(clean - exact) <= bound)
    # a dropped term, a transposed operand or a wrong sign would be far outside the bound
    assert np.abs(clean - exact).max() < 1e-3


def test_noisy_logits(orc):
    """H = fma(eps, softplus(x W_noise), clean); checked against fp64 with a
    rounding bound, and sigma against the fp64 softplus of the exact dot."""
    cfg = scaled(CONFIGS["noisy_top4"], T=48, E=16)
    inp = make_inputs(cfg, with_weights=False)
    clean, sigma, H = orc.gate_logits(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w_noise"],
                                      inp["noise"], "bf16")
    xf = _widen(inp["x"]).astype(np.float64)
    zn = xf @ _widen(inp["w_noise"]).astype(np.float64)
    sp_ref = np.logaddexp(0.0, zn)
    # noise-dot rounding (<= 1e-4 here) moves softplus by at most that much (1-Lipschitz)
    assert np.abs(sigma - sp_ref).max() < 2e-4
    h_ref = clean.astype(np.float64) + inp["noise"].astype(np.float64) * sigma.astype(np.float64)
    assert np.all(np.abs(H - h_ref) <= np.spacing(np.abs(h_ref).astype(np.float32)))
    clean_ref = xf @ _widen(inp["w_gate"]).astype(np.float64) + inp["gate_bias"]
    assert np.abs(clean - clean_ref).max() < 1e-3
    assert np.all(sigma > 0)


# --------------------------------------------------------------------------
# top-k order
# --------------------------------------------------------------------------
def _tie_heavy_H(T, E, seed):
    rng = np.random.default_rng(seed)
    H = np.round(rng.standard_normal((T, E)) * 2) / 2  # many exact ties
    H[::7] = 0.0  # whole rows tied
    H[1::11, :] = -0.0
    H[2::13, : max(1, E // 2)] = 0.0  # mixed +0/-0 ties
    return H.astype(np.float32)


@pytest.mark.parametrize("E,kk", [(1, 1), (4, 2), (8, 3), (16, 5), (64, 9), (256, 5)])
def test_topk_order_matches_numpy_stable_argsort(orc, E, kk):
    H = _tie_heavy_H(200, E, seed=E)
    got = orc.topk_order(H, kk)
    ref = np.argsort(-H, axis=1, kind="stable")[:, :kk]
    assert np.array_equal(got, ref)


def test_topk_set_is_lexicographically_smallest_max_sum_subset(orc):
    rng = np.random.default_rng(9)
    for E in range(1, 7):
        for k in range(1, min(E, 3) + 1):
            H = np.round(rng.standard_normal((40, E)) * 2).astype(np.float32)
            got = orc.topk_order(H, k)
            for t in range(H.shape[0]):
                best = None
                for sub in itertools.combinations(range(E), k):  # lexicographic order
                    s = sum(Fraction(float(H[t, e])) for e in sub)
                    if best is None or s > best[0]:
                        best = (s, sub)
                assert tuple(sorted(got[t])) == best[1]


# --------------------------------------------------------------------------
# gate values
# --------------------------------------------------------------------------
def test_gates_renormalised_and_raw(orc):
    rng = np.random.default_rng(10)
    T, E, k = 300, 12, 3
    H = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    idx = orc.topk_order(H, k)
    g_ren, prob = orc.gates(H, idx, True)
    g_raw, prob2 = orc.gates(H, idx, False)
    p_ref = softmax(H.astype(np.float64), axis=1)
    assert np.allclose(prob, p_ref, rtol=1e-13, atol=0)
    assert np.array_equal(prob, prob2)
    # raw gates are the full-softmax probabilities of the kept experts
    assert np.allclose(g_raw, np.take_along_axis(p_ref, idx, 1), rtol=1e-13, atol=0)
    # softmax over the kept logits == kept probabilities renormalised, sums to 1
    kept = np.take_along_axis(p_ref, idx, 1)
    assert np.allclose(g_ren, kept / kept.sum(1, keepdims=True), rtol=1e-12, atol=0)
    assert np.allclose(g_ren.sum(1), 1.0, rtol=0, atol=1e-14)
    # KeepTopK then Softmax: -inf outside the kept set
    masked = np.full_like(H, -np.inf, dtype=np.float64)
    np.put_along_axis(masked, idx, np.take_along_axis(H, idx, 1).astype(np.float64), 1)
    assert np.allclose(g_ren, np.take_along_axis(softmax(masked, axis=1), idx, 1), rtol=1e-12)
    # gates are ordered like the logits
    assert np.all(np.diff(g_ren, axis=1) <= 0)


def test_top1_raw_gate_at_least_one_over_E(orc):
    rng = np.random.default_rng(11)
    H = rng.standard_normal((500, 128)).astype(np.float32)
    idx = orc.topk_order(H, 1)
    g, _ = orc.gates(H, idx, False)
    assert np.all(g >= 1.0 / 128 - 1e-15)
    g1, _ = orc.gates(H, idx, True)
    assert np.all(g1 == 1.0)


# --------------------------------------------------------------------------
# capacity and dispatch
# --------------------------------------------------------------------------
def test_capacity_values(orc):
    assert orc.capacity(16384, 128, 1, 1.25) == 160  # switch_top1
    assert orc.capacity(32768, 64, 2, 2.0) == 2048  # gshard_top2
    assert orc.capacity(100, 3, 1, 1.0) == 34  # ceil(33.33)
    assert orc.capacity(100, 3, 1, 0.0) == -1
    assert orc.capacity(100, 3, 1, 1.0, explicit=7) == 7
    assert orc.capacity(100, 3, 1, 0.0, explicit=0) == 0


def _dispatch_reference(idx, E, C):
    """Independent statement: stable argsort of the flattened expert ids gives
    the (expert, token) order; an assignment's rank is its position within its
    expert's run."""
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    start = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty_like(flat)
    rank[order] = np.arange(flat.size) - start[flat[order]]
    keep = rank < C if C >= 0 else np.ones_like(flat, bool)
    kept = np.minimum(counts, C) if C >= 0 else counts
    offsets = np.concatenate([[0], np.cumsum(kept)])
    slot = np.where(keep, offsets[flat] + rank, -1)
    return counts, kept, offsets, slot.reshape(idx.shape)


@pytest.mark.parametrize("T,E,k,C", [(1, 1, 1, -1), (50, 4, 2, 10), (1000, 16, 3, 150), (1000, 16, 3, 0),
                                     (333, 7, 1, 40), (2048, 128, 1, 20), (5, 8, 8, 3)])
def test_dispatch_matches_stable_argsort_and_invariants(orc, T, E, k, C):
    rng = np.random.default_rng(T + E)
    H = rng.standard_normal((T, E)).astype(np.float32)
    H[:, 0] += 1.0  # a hot expert so capacity binds
    idx = orc.topk_order(H, k)
    out = orc.dispatch(idx, E, C)
    counts, kept, offsets, slot = _dispatch_reference(idx, E, C)
    assert np.array_equal(out["counts_routed"], counts)
    assert np.array_equal(out["counts_kept"], kept)
    assert np.array_equal(out["offsets"], offsets)
    assert np.array_equal(out["slot_dest"], slot)
    # invariants: totals, drops, bijection, (expert, token) order
    assert out["counts_routed"].sum() == T * k
    drops = int((out["slot_dest"] < 0).sum())
    assert out["counts_kept"].sum() == T * k - drops == out["R"]
    live = out["slot_dest"][out["slot_dest"] >= 0]
    assert np.array_equal(np.sort(live), np.arange(out["R"]))
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    assert np.array_equal(out["row_src"][out["slot_dest"][out["slot_dest"] >= 0]], tok[out["slot_dest"] >= 0])
    row_exp = np.repeat(np.arange(E), out["counts_kept"])
    keys = row_exp.astype(np.int64) * (T + 1) + out["row_src"]
    assert np.all(np.diff(keys) > 0)


def test_dispatch_sequential_simulation(orc):
    """Brute-force token-order walk with a per-expert fill counter."""
    rng = np.random.default_rng(12)
    T, E, k, C = 400, 6, 2, 70
    idx = orc.topk_order(rng.standard_normal((T, E)).astype(np.float32), k)
    out = orc.dispatch(idx, E, C)
    fill = [0] * E
    ranks = {}
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            ranks[(t, s)] = fill[e]
            fill[e] += 1
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            r = ranks[(t, s)]
            want = int(out["offsets"][e]) + r if r < C else -1
            assert out["slot_dest"][t, s] == want


def _slot_major_walk(idx, E, C):
    """First-choice priority by brute force: serve every token's first choice
    (in token order), then every token's second choice, and so on; each
    assignment takes its expert's next rank; rank >= C is dropped."""
    T, k = idx.shape
    fill = [0] * E
    rank = {}
    for s in range(k):
        for t in range(T):
            e = int(idx[t, s])
            rank[(t, s)] = fill[e]
            fill[e] += 1
    return fill, rank


@pytest.mark.parametrize("T,E,k,C", [(400, 6, 2, 70), (300, 5, 3, 40), (64, 8, 8, 5), (50, 4, 1, 7),
                                     (200, 9, 2, -1), (100, 3, 2, 0)])
def test_dispatch_first_choice_priority_walk(orc, T, E, k, C):
    rng = np.random.default_rng(T * 7 + k)
    H = rng.standard_normal((T, E)).astype(np.float32)
    H[:, 1] += 1.5  # a hot expert: many first choices land on it, capacity binds there first
    idx = orc.topk_order(H, k)
    out = orc.dispatch(idx, E, C, slot_major=True)
    fill, rank = _slot_major_walk(idx, E, C)
    assert list(out["counts_routed"]) == fill
    kept = [min(c, C) if C >= 0 else c for c in fill]
    assert list(out["counts_kept"]) == kept
    assert list(out["offsets"]) == list(np.concatenate([[0], np.cumsum(kept)]))
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            r = rank[(t, s)]
            want = int(out["offsets"][e]) + r if (C < 0 or r < C) else -1
            assert out["slot_dest"][t, s] == want
            if want >= 0:
                assert out["row_src"][want] == t
    # the defining property: a first choice is dropped only if its expert's capacity
    # is filled by first choices alone
    first = idx[:, 0]
    n_first = np.bincount(first, minlength=E)
    dropped_first = out["slot_dest"][:, 0] < 0
    if C >= 0:
        assert np.all(n_first[first[dropped_first]] > C)
    else:
        assert not dropped_first.any()


def test_first_choice_priority_equals_token_order_for_top1(orc):
    rng = np.random.default_rng(9)
    idx = orc.topk_order(rng.standard_normal((500, 7)).astype(np.float32), 1)
    a = orc.dispatch(idx, 7, 40)
    b = orc.dispatch(idx, 7, 40, slot_major=True)
    for key in ("counts_kept", "offsets", "slot_dest", "row_src"):
        assert np.array_equal(a[key], b[key])


def test_zero_gate_weights_route_everything_to_expert_zero(orc):
    """W_g = 0: all logits tie, the lower index wins, so every token picks
    expert 0 first; with capacity C exactly C are kept, T - C dropped."""
    T, d, E, C = 500, 16, 8, 123
    x = _bf16(np.random.default_rng(13).standard_normal((T, d)))
    w = np.zeros((d, E), np.uint16)
    _, _, H = orc.gate_logits(x, w, dtype="bf16")
    idx = orc.topk_order(H, 1)
    assert np.all(idx == 0)
    out = orc.dispatch(idx, E, C)
    assert out["counts_kept"][0] == C and out["counts_kept"][1:].sum() == 0
    assert (out["slot_dest"] < 0).sum() == T - C
    assert np.array_equal(out["slot_dest"][:C, 0], np.arange(C))
    g, _ = orc.gates(H, idx, False)
    assert np.allclose(g, 1.0 / E, rtol=1e-15)


# --------------------------------------------------------------------------
# balancing losses
# --------------------------------------------------------------------------
def test_switch_aux_closed_forms(orc):
    E, T, k = 8, 64, 1
    rng = np.random.default_rng(14)
    counts = rng.multinomial(T * k, np.ones(E) / E).astype(np.int32)
    # uniform probabilities: exactly 1 for any routed fractions
    a = orc.aux(T, k, counts, np.full(E, T / E), np.ones(E))
    assert abs(a[0] - 1.0) < 1e-15
    # uniform routed fractions: exactly 1 for any probabilities
    p = rng.dirichlet(np.ones(E), size=T).sum(0)
    a = orc.aux(T, k, np.full(E, T * k // E, np.int32), p, np.ones(E))
    assert abs(a[0] - 1.0) < 1e-14
    # everything on expert 0 with probability q: E * q
    q = 0.7
    ps = np.zeros(E)
    ps[0] = q * T
    c = np.zeros(E, np.int32)
    c[0] = T
    a = orc.aux(T, k, c, ps, np.ones(E))
    assert abs(a[0] - E * q) < 1e-14


def test_cv_squared_closed_forms(orc):
    E = 10
    c = np.ones(E, np.int32)
    a = orc.aux(E, 1, c, np.ones(E), np.full(E, 3.0), np.full(E, 2.0))
    assert a[1] == 0.0 and a[2] == 0.0
    one = np.zeros(E)
    one[3] = 5.0
    a = orc.aux(E, 1, c, np.ones(E), one, one)
    assert abs(a[1] - (E - 1)) < 1e-12 and abs(a[2] - (E - 1)) < 1e-12
    a = orc.aux(1, 1, np.ones(1, np.int32), np.ones(1), np.ones(1))
    assert a[1] == 0.0 and np.isnan(a[2])
    v = np.random.default_rng(15).uniform(0.1, 2, E)
    a = orc.aux(E, 1, c, np.ones(E), v)
    assert abs(a[1] - np.var(v) / np.mean(v) ** 2) < 1e-13


def test_load_estimator_matches_monte_carlo(orc):
    """P(x,i) is the probability that expert i is in the top k when only its own
    noise is re-drawn (the smooth estimator of the Load-Balancing-Losses
    section). Check each token's P(x,i) against M re-draws, within 4 sigma."""
    rng = np.random.default_rng(16)
    T, E, k, M = 6, 7, 2, 40000
    clean = rng.standard_normal((T, E)).astype(np.float32)
    sigma = rng.uniform(0.3, 1.5, (T, E)).astype(np.float32)
    eps = rng.standard_normal((T, E)).astype(np.float32)
    H = (clean + eps * sigma).astype(np.float32)
    order = orc.topk_order(H, k + 1)
    for t in range(T):
        for i in range(E):
            ld = orc.load(clean[t:t + 1], sigma[t:t + 1], H[t:t + 1], order[t:t + 1], k)
            p_oracle = ld[i]
            others = np.delete(H[t].astype(np.float64), i)
            kth = np.sort(others)[::-1][k - 1]
            draws = clean[t, i] + rng.standard_normal(M) * sigma[t, i]
            p_mc = np.mean(draws > kth)
            assert abs(p_oracle - p_mc) <= 4 * np.sqrt(0.25 / M) + 1e-12
            # and the closed form with scipy's normal cdf
            assert abs(p_oracle - ndtr((clean[t, i] - kth) / sigma[t, i])) < 1e-6


def test_load_all_experts_kept_is_one(orc):
    T, E = 5, 4
    rng = np.random.default_rng(17)
    clean = rng.standard_normal((T, E)).astype(np.float32)
    sigma = np.ones((T, E), np.float32)
    H = clean.copy()
    order = orc.topk_order(H, E)
    ld = orc.load(clean, sigma, H, order, E)
    assert np.array_equal(ld, np.full(E, float(T)))
