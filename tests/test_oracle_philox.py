"""Pins of the oracle's Philox4x32-10 and of its Bernoulli draws (CPU)."""
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox, poissoncomp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _kat())
def test_known_answer_vectors(row):
    c, k, x = row[:4], row[4:6], row[6:]
    out = philox.philox4x32(*c, *k)
    assert [int(v) for v in out] == x


def test_vectorised_matches_scalar():
    ctr = np.arange(50, dtype=np.uint64) * 7919 + 3
    vec = philox.philox4x32(ctr, 5, 6, 7, 11, 13)
    for j, c in enumerate(ctr):
        sc = philox.philox4x32(int(c), 5, 6, 7, 11, 13)
        assert [int(a[j]) for a in vec] == [int(v) for v in sc]


def test_uniform53_range_and_uniformity():
    u = philox.uniform53(np.arange(200_000), 3, 1, 0, 12345)
    assert u.min() >= 0.0 and u.max() < 1.0
    # 53-bit lattice values
    assert np.all(u * 2.0 ** 53 == np.floor(u * 2.0 ** 53))
    hist, _ = np.histogram(u, bins=100, range=(0.0, 1.0))
    chi2 = stats.chisquare(hist)
    assert chi2.pvalue > 1e-4
    # neighbouring counters are uncorrelated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.01


def test_streams_differ_by_every_counter_word_and_seed():
    base = philox.uniform53(np.arange(64), 0, 0, 0, 7)
    for args in [(1, 0, 0, 7), (0, 1, 0, 7), (0, 0, 1, 7), (0, 0, 0, 8), (0, 0, 0, 7 + (1 << 32))]:
        other = philox.uniform53(np.arange(64), *args)
        assert not np.any(other == base)


def test_bernoulli_frequency_matches_r():
    """E[Z_i] = r_i (Poisson sampling, independent Bernoulli draws): frequencies over
    4000 seeds lie inside 99.9% Clopper-Pearson intervals."""
    r = np.array([0.5, 0.01, 0.3, 0.999, 0.2, 0.05, 0.7, 0.9], dtype=np.float64)
    nseed = 4000
    counts = np.zeros(r.size)
    for s in range(nseed):
        counts += poissoncomp.draw(r, 0, 0, 0, s)
    for c, p in zip(counts, r):
        lo = stats.beta.ppf(0.0005, c, nseed - c + 1) if c > 0 else 0.0
        hi = stats.beta.ppf(0.9995, c + 1, nseed - c) if c < nseed else 1.0
        assert lo <= p <= hi, (c, p)
