"""Pins for the oracle's counter-based standard-normal noise (the
StandardNormal() draw of "Noisy Top-K Gating" on the Shazeer et al. summary
page, made reproducible: Philox4x32-10 words, Box-Muller in fp32 from
correctly rounded operations).

* the transform against the fp64 closed form sqrt(-2 ln u1) cos(2 pi u2) on
  the same uniforms (numpy's log / cos / sqrt), within a few ulp;
* the counter RNG by its defining properties: a bijection of the 128-bit
  counter for a fixed key (no output collisions), full avalanche (one flipped
  counter or key bit flips half of the 128 output bits), uniform bytes in
  every output word, independent streams per key, and the counter addressing
  (row offset, row high word, column);
* the normal stream by its distribution: moments, tail mass and a
  Kolmogorov-Smirnov test against scipy's normal CDF.
"""

import numpy as np
import pytest
from scipy import stats


def _uniforms(w0, w1):
    u1 = ((w0 >> 8).astype(np.float64) + 1.0) * 2.0 ** -24
    u2 = (w1 >> 8).astype(np.float64) * 2.0 ** -24
    return u1, u2


def test_transform_matches_fp64_box_muller(orc):
    rng = np.random.default_rng(0)
    w = rng.integers(0, 2 ** 32, size=(400_000, 2), dtype=np.uint64).astype(np.uint32)
    # the extremes of both uniforms and the branch points of the cosine folding
    edge = np.array([[0, 0], [0xFFFFFFFF, 0xFFFFFFFF], [0, 0x40000000], [0, 0x20000000], [0, 0x80000000],
                     [0, 0x60000000], [0xFFFFFF00, 0xC0000000], [0x100, 0x10000000]], np.uint32)
    w = np.concatenate([w, edge])
    z = orc.normal_from_words(w).astype(np.float64)
    u1, u2 = _uniforms(w[:, 0], w[:, 1])
    ref = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    # radius (sqrt of ~2 ulp ln) and angle (fp32(2 pi), one rounding of the product) add a few ulp;
    # near the cosine's zeros the angle's rounding dominates: absolute 2 * 2^-24 * 2 pi * radius
    bound = 6 * ulp + np.sqrt(-2.0 * np.log(u1)) * 2.0 ** -21
    bad = np.abs(z - ref) > bound
    assert not bad.any(), (w[bad][:5], z[bad][:5], ref[bad][:5])
    assert z[-8] == pytest.approx(np.sqrt(2 * 24 * np.log(2.0)), rel=1e-6)  # u1 = 2^-24, u2 = 0


def test_philox_is_a_bijection_with_full_avalanche(orc):
    w = orc.philox_words(7, 2048, 512).reshape(-1, 4)  # 1M distinct counters
    as_bytes = np.ascontiguousarray(w).view(np.dtype((np.void, 16)))
    assert np.unique(as_bytes).size == w.shape[0], "two counters gave the same output block"
    # flipping one counter bit (column 0 -> 1, row r -> r ^ 2^j) changes ~64 of 128 bits
    base = orc.philox_words(7, 1, 64, row0=1000)[0]  # columns 0..63 of row 1000
    pop = np.unpackbits((base[:-1] ^ base[1:]).view(np.uint8)).reshape(63, -1).sum(1)
    assert 54 < pop.mean() < 74 and pop.min() > 30
    rows = np.array([orc.philox_words(7, 1, 1, row0=1000 ^ (1 << j))[0, 0] for j in range(40)])
    pop = np.unpackbits((rows ^ orc.philox_words(7, 1, 1, row0=1000)[0, 0]).view(np.uint8)).reshape(40, -1).sum(1)
    assert 54 < pop.mean() < 74 and pop.min() > 30
    # one key bit
    k = np.array([orc.philox_words(7 ^ (1 << j), 1, 1)[0, 0] for j in range(64)])
    pop = np.unpackbits((k ^ orc.philox_words(7, 1, 1)[0, 0]).view(np.uint8)).reshape(64, -1).sum(1)
    assert 54 < pop.mean() < 74 and pop.min() > 30


def test_philox_output_bytes_are_uniform(orc):
    w = orc.philox_words(123, 1024, 256)
    for word in range(4):
        b = np.ascontiguousarray(w[:, :, word]).reshape(-1).view(np.uint8)
        counts = np.bincount(b, minlength=256)
        chi2 = ((counts - b.size / 256) ** 2 / (b.size / 256)).sum()
        assert stats.chi2.sf(chi2, 255) > 1e-4, (word, chi2)


def test_counter_addressing_and_streams(orc):
    a = orc.normal_noise(99, 64, 48)
    b = orc.normal_noise(99, 16, 48, row0=40)
    assert np.array_equal(a[40:56], b)  # element (row, col) does not depend on the call's first row
    hi = orc.normal_noise(99, 2, 48, row0=(1 << 32) + 40)
    assert not np.array_equal(hi, a[40:42])  # the row's high word is part of the counter
    c = orc.normal_noise(100, 64, 48)
    assert np.abs(np.corrcoef(a.ravel(), c.ravel())[0, 1]) < 0.05
    assert not np.array_equal(a[:, 0], a[:, 1])


def test_noise_is_standard_normal(orc):
    z = orc.normal_noise(2024, 4096, 256).astype(np.float64).ravel()  # 1M draws
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    assert abs(stats.skew(z)) < 5 * np.sqrt(6.0 / n)
    assert abs(stats.kurtosis(z)) < 5 * np.sqrt(24.0 / n)
    tail = np.mean(np.abs(z) > 3.0)
    p3 = 2 * stats.norm.sf(3.0)
    assert abs(tail - p3) < 5 * np.sqrt(p3 / n)
    assert stats.kstest(z[:200_000], "norm").pvalue > 1e-3
