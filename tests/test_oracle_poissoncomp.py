"""Pins of the oracle's PoissonComp (eq. 3 water-filling, H/L partition, sample)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from long_context_decode_kvfetch_amd import synth
from oracle import poissoncomp as pc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases():
    cases = []
    with open(os.path.join(GOLDEN, "waterfill_hand.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                eta, tau, r, c = [p.strip() for p in line.split("|")]
                cases.append((float(eta), [float(x) for x in tau.split()],
                              [float(x) for x in r.split()], float(c)))
    return cases


@pytest.mark.parametrize("case", _hand_cases())
def test_hand_solved_examples(case):
    eta, tau, r_exp, c_exp = case
    r, _, c = pc.inclusion_probabilities(np.array(tau, np.float32), 0, 0, eta)
    np.testing.assert_allclose(r, r_exp, rtol=1e-15, atol=0)
    if c:
        assert math.isclose(c * 2.0 ** 40, c_exp, rel_tol=1e-15)


def _exact_waterfill(q, b_rem):
    """Exact rational water level for sum_i min(1, c q_i) = b_rem (q as integers)."""
    order = sorted(range(len(q)), key=lambda j: -q[j])
    B = Fraction(b_rem)
    S = sum(q)
    for m, j in enumerate(order):
        c = (B - m) / S if S else None
        if c is not None and B - m > 0 and c * q[j] < 1 and (m == 0 or c * q[order[m - 1]] >= 1):
            return m, c
        S -= q[j]
    return None, None


@pytest.mark.parametrize("seed,n,eta,kind", [(0, 300, 0.125, "beta"), (1, 2000, 1 / 16, "beta"),
                                             (2, 1000, 0.3, "uniform"), (3, 777, 0.05, "zipf")])
def test_matches_exact_rational_waterfill(seed, n, eta, kind):
    rng = np.random.default_rng(seed)
    if kind == "beta":
        tau = rng.beta(0.3, 3.0, n).astype(np.float32)
    elif kind == "uniform":
        tau = rng.random(n).astype(np.float32)
    else:
        tau = ((rng.permutation(n) + 1.0) ** -1.1).astype(np.float32)
    n_sink, n_local = 4, 16
    r, m_star, c = pc.inclusion_probabilities(tau, n_sink, n_local, eta)
    free = np.arange(n_sink, n - n_local)
    q = pc.quantize(tau[free])
    b_rem = eta * n - (n_sink + n_local)
    m_ex, c_ex = _exact_waterfill(q, b_rem)
    assert m_ex == m_star
    assert abs(c - float(c_ex)) <= 2.0 ** -52 * float(c_ex)
    # every r_i equals min(1, c q_i) of the exact level up to one rounding
    for j, i in enumerate(free):
        want = min(Fraction(1), c_ex * q[j])
        assert abs(r[i] - float(want)) <= 2.0 ** -51 * float(want) + 0.0
    # and, against the unquantised tau, to the scale of the quantisation step
    c_tau = float(c_ex) * 2.0 ** 40
    r_tau = np.minimum(1.0, c_tau * tau[free].astype(np.float64))
    assert np.all(np.abs(r[free] - r_tau) <= 2.0 ** -40 * c_tau + 1e-15)


@pytest.mark.parametrize("eta", [1 / 8, 1 / 16, 1 / 32, 0.3, 0.9])
def test_budget_is_spent_exactly_and_r_is_monotone(eta):
    rng = np.random.default_rng(11)
    n = 5000
    tau = rng.beta(0.3, 3.0, n).astype(np.float32)
    r, m_star, _ = pc.inclusion_probabilities(tau, 4, 128, eta)
    assert abs(r.sum() - eta * n) <= 1e-9 * eta * n
    assert np.all((r >= 0) & (r <= 1))
    free = np.arange(4, n - 128)
    o = np.argsort(tau[free], kind="stable")
    assert np.all(np.diff(r[free][o]) >= 0)          # r non-decreasing in tau
    assert np.all(r[:4] == 1) and np.all(r[-128:] == 1)
    assert int(np.sum(r[free] == 1.0)) == m_star


def test_edge_cases():
    tau = np.linspace(0.1, 1.0, 100).astype(np.float32)
    with pytest.raises(pc.BudgetError):
        pc.inclusion_probabilities(tau, 8, 8, 0.1)      # 10 < 16 forced
    r, _, _ = pc.inclusion_probabilities(tau, 5, 5, 0.1)  # budget exactly the forced tokens
    assert np.all(r[5:95] == 0.0) and r.sum() == 10
    r, _, _ = pc.inclusion_probabilities(tau, 5, 5, 1.0)  # eta = 1: everything kept
    assert np.all(r == 1.0)
    tz = tau.copy()
    tz[40:60] = 0.0
    r, _, _ = pc.inclusion_probabilities(tz, 5, 5, 0.3)
    assert np.all(r[40:60] == 0.0)
    assert abs(r.sum() - 30) <= 1e-12
    with pytest.raises(ValueError):
        pc.inclusion_probabilities(np.array([0.5, 1.5], np.float32), 0, 0, 0.5)


def test_sample_contains_H_and_expected_size():
    wl = synth.gqa_layer(seed=3, n=8192, steps=1, hkv=1)
    s = wl.seqs[0]
    sizes = []
    for seed in range(40):
        c = pc.compress_head(s.tau[0], 4, 128, 1 / 16, 0, 0, 0, seed)
        assert np.all(c.resident[c.r >= 1.0])
        assert np.all(np.diff(c.piv_idx) > 0)
        sizes.append(c.piv_idx.size)
    # E|H u S| = sum r = eta n; sd <= sqrt(eta n)
    assert abs(np.mean(sizes) - 8192 / 16) < 4 * math.sqrt(512 / 40)
