"""Pins for the oracle's canonical softplus and its exp / log1p pieces.

The noise scale of noisy top-k gating is Softplus((x W_noise)_i) (Shazeer et
al. summary page, "Methode", "Noisy Top-K Gating"). The oracle defines it from
basic IEEE fp32 operations; these tests tie that definition to the true
function (fp64 numpy/math) within a few units in the last place.
"""

import math

import numpy as np
import pytest

ULP1 = float(np.spacing(np.float32(1.0)))  # 2^-23


def _ulps(got, ref):
    got = got.astype(np.float64)
    scale = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return np.abs(got - ref) / scale


def _dense_f32(lo, hi, n, seed=0):
    rng = np.random.default_rng(seed)
    a = rng.uniform(lo, hi, n).astype(np.float32)
    grid = np.linspace(lo, hi, n // 4, dtype=np.float32)
    return np.concatenate([a, grid])


def test_exp_nonpos_matches_math_exp(orc):
    y = _dense_f32(-87.0, 0.0, 400_000)
    got = orc.exp_nonpos(y)
    ref = np.exp(y.astype(np.float64))
    assert _ulps(got, ref).max() <= 2.0


def test_exp_nonpos_special_points(orc):
    got = orc.exp_nonpos(np.array([0.0, -0.0, -87.5, -100.0, -1e30], np.float32))
    assert got[0] == 1.0 and got[1] == 1.0
    assert np.all(got[2:] == 0.0)  # defined as zero below -87
    # exp(-ln 2 * n) lands on powers of two up to rounding of the argument
    for n in range(0, 120, 7):
        y = np.float32(-n * math.log(2.0))
        g = float(orc.exp_nonpos(np.array([y], np.float32))[0])
        assert abs(g - math.exp(float(y))) <= 2 * np.spacing(np.float32(math.exp(float(y))))


def test_log1p_unit_matches_numpy(orc):
    v = _dense_f32(0.0, 1.0, 400_000, seed=1)
    v = np.concatenate([v, np.array([0.0, 1.0, 1e-30, 1e-8, 0.5], np.float32)])
    got = orc.log1p_unit(v)
    ref = np.log1p(v.astype(np.float64))
    nz = ref > 0
    assert _ulps(got[nz], ref[nz]).max() <= 3.0
    assert got[v == 0.0][0] == 0.0


@pytest.mark.parametrize("lo,hi", [(-100.0, -20.0), (-20.0, 0.0), (0.0, 20.0), (20.0, 100.0)])
def test_softplus_few_ulp(orc, lo, hi):
    z = _dense_f32(lo, hi, 400_000, seed=2)
    got = orc.softplus(z)
    zd = z.astype(np.float64)
    ref = np.where(zd > 0, zd + np.log1p(np.exp(-zd)), np.log1p(np.exp(zd)))
    big = ref > 1e-37  # below that the definition returns 0 (absolute error < 2e-38)
    assert _ulps(got[big], ref[big]).max() <= 4.0
    assert np.all(np.abs(got[~big] - ref[~big]) < 2e-38)


def test_softplus_identities(orc):
    # softplus(0) = ln 2; softplus(z) - softplus(-z) = z; monotone; z > 20 returns z
    assert abs(float(orc.softplus(np.float32(0.0))[0]) - math.log(2.0)) <= ULP1
    z = np.linspace(-15, 15, 30001, dtype=np.float32)
    sp, spn = orc.softplus(z), orc.softplus(-z)
    assert np.max(np.abs((sp.astype(np.float64) - spn) - z)) <= 16 * ULP1 * 16
    zs = np.sort(_dense_f32(-90, 90, 200_000, seed=3))
    s = orc.softplus(zs)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)
    big = np.array([20.0001, 25.0, 1e4], np.float32)
    assert np.array_equal(orc.softplus(big), big)
