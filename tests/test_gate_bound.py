"""The error bound behind the certified MFMA gate, checked on the CPU.

The bf16 layers compute their gate logits with MFMAs and keep a token's top-k
only if every gap among its top-(k+1) values exceeds twice the bound

    B = 100 u (Q + S) (1 + 256 u M),   u = 2^-24,  M = ceil(d / 32),
    S = sum_j |x_j w_j|,  Q = sum over the M k-steps of |accumulator after the step|,

on the distance between the MFMA value and the canonical value (an fp32
fma chain from +0 over j ascending). The derivation assumes each 32-term MFMA
step is off by at most 64 u (|accumulator before| + sum of the step's |terms|).
These tests emulate accumulations that satisfy that model -- one rounding per
step, rounding after every add in other orders, truncation instead of rounding
-- on random, heavy-tailed and cancelling inputs, and check that the
canonical value always lies within B of them, with room to spare. The GPU
parity tests then check the routing itself against the oracle in every gate
mode.
"""

from __future__ import annotations

import numpy as np
import pytest

from synthetic import bf16_bits_to_f32, f32_to_bf16_bits

U = 2.0 ** -24


def _bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, np.float32)))


def _canonical(x, w):
    """fp32 fma chain from +0, j ascending (products of bf16 values are exact in fp32)."""
    s = np.float32(0.0)
    for xj, wj in zip(x, w):
        s = np.float32(s + np.float32(xj) * np.float32(wj))
    return float(s)


def _trunc32(v):
    """Round toward zero to fp32."""
    f = np.float32(v)
    if abs(float(f)) > abs(v):
        f = np.nextafter(f, np.float32(0.0))
    return f


def _mfma_models(x, w):
    """Accumulator values after each 32-term step under several models, and the final values."""
    p = x.astype(np.float64) * w.astype(np.float64)
    out = {}
    # one rounding per step (exact inner sum)
    acc, hist = np.float32(0.0), []
    for j0 in range(0, len(p), 32):
        acc = np.float32(float(acc) + p[j0:j0 + 32].sum())
        hist.append(float(acc))
    out["exact_inner"] = (float(acc), hist)
    # pairwise tree inside the step, fp32 rounding at every add
    acc, hist = np.float32(0.0), []
    for j0 in range(0, len(p), 32):
        v = [np.float32(t) for t in p[j0:j0 + 32]]
        while len(v) > 1:
            v = [np.float32(v[i] + v[i + 1]) if i + 1 < len(v) else v[i] for i in range(0, len(v), 2)]
        acc = np.float32(acc + v[0])
        hist.append(float(acc))
    out["pairwise"] = (float(acc), hist)
    # sequential with truncation after every add
    acc, hist = np.float32(0.0), []
    for j0 in range(0, len(p), 32):
        for t in p[j0:j0 + 32]:
            acc = _trunc32(float(acc) + t)
        hist.append(float(acc))
    out["truncating"] = (float(acc), hist)
    return out


def _bound(x, w, hist):
    S = float(np.abs(x.astype(np.float64) * w.astype(np.float64)).sum())
    Q = float(np.abs(np.array(hist)).sum())
    M = len(hist)
    return 100.0 * U * (Q + S) * (1.0 + 256.0 * U * M)


def _cases(rng, d):
    yield _bf16(rng.standard_normal(d)), _bf16(rng.standard_normal(d) * 0.05)
    yield _bf16(rng.standard_t(2, d)), _bf16(rng.standard_t(2, d))  # heavy tails
    a = _bf16(rng.standard_normal(d))
    yield np.concatenate([a[: d // 2], a[: d // 2]]), np.concatenate([np.ones(d // 2), -np.ones(d // 2)]).astype(np.float32)
    big = _bf16(rng.standard_normal(d) * np.where(rng.random(d) < 0.05, 1e3, 1.0))
    yield big, _bf16(rng.standard_normal(d))  # a few dominant terms, large cancellations


@pytest.mark.parametrize("d", [32, 96, 768])
def test_canonical_value_within_the_bound_of_every_model(d):
    rng = np.random.default_rng(d)
    worst = 0.0
    for _ in range(6 if d == 768 else 20):
        for x, w in _cases(rng, d):
            c = _canonical(x, w)
            for name, (v, hist) in _mfma_models(x, w).items():
                B = _bound(x, w, hist)
                assert abs(v - c) <= B, (name, d, v, c, B)
                if B > 0:
                    worst = max(worst, abs(v - c) / B)
    assert worst < 0.5  # the bound is not tight on these inputs: the certificate has margin


def test_bound_separates_certified_gaps():
    """A gap of more than 2B between two MFMA values fixes their canonical order."""
    rng = np.random.default_rng(7)
    d = 256
    for _ in range(50):
        x = _bf16(rng.standard_normal(d))
        w1, w2 = _bf16(rng.standard_normal(d) * 0.1), _bf16(rng.standard_normal(d) * 0.1)
        v1, h1 = _mfma_models(x, w1)["truncating"]
        v2, h2 = _mfma_models(x, w2)["truncating"]
        B = max(_bound(x, w1, h1), _bound(x, w2, h2))
        c1, c2 = _canonical(x, w1), _canonical(x, w2)
        if v1 - v2 > 2 * B:
            assert c1 > c2
        if v2 - v1 > 2 * B:
            assert c2 > c1
