"""Pins of the oracle's growing-cache step (oracle/poissoncomp.py: append_token).

The pages compress the cache once, at prefill; tokens appended during decode are a
reading (the appended token joins the local window, the token leaving it gets the
prefill's rule and water level and its own Philox draw).  These tests pin what that
reading implies: budget bookkeeping, agreement with the prefill's eq. (3) rule, the
draw frequencies, each branch of the rule, and that a grown state decodes like any
compressed cache (exact attention over all tokens when every L token is fetched)."""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

from oracle import api as oapi
from oracle import poissoncomp as pc


def _comp(n=64, n_sink=2, n_local=4, eta=0.25, seed=0, tau=None):
    if tau is None:
        tau = np.random.default_rng(seed).random(n).astype(np.float32)
    return pc.compress_head(tau, n_sink, n_local, eta, 0, 0, 0, seed), tau


def test_budget_grows_by_the_departing_probability():
    comp, _ = _comp()
    rng = np.random.default_rng(5)
    for _ in range(20):
        n = len(comp.r)
        new = pc.append_token(comp, float(rng.random()), 2, 4, 0, 0, 0, 0)
        t = n - 4
        assert len(new.r) == n + 1 and new.r[-1] == 1.0 and new.resident[-1]
        assert comp.r[t] == 1.0                       # it was in the local window
        before = sum(Fraction(float(x)) for x in comp.r)
        after = sum(Fraction(float(x)) for x in new.r)
        assert after == before + Fraction(float(new.r[t]))   # t: 1 -> r_t, new token: +1
        assert np.array_equal(new.piv_idx, np.flatnonzero(new.resident))
        assert np.array_equal(new.r[:t], comp.r[:t]) and np.array_equal(new.resident[:t], comp.resident[:t])
        comp = new


def test_departing_token_gets_the_prefill_rule():
    """A token leaving the window with the score of a non-forced prefill token gets
    exactly that token's r (eq. 3 with the prefill's water level), saturated or not."""
    n = 300
    rho = np.random.default_rng(3).permutation(n) + 1
    tau = (rho.astype(np.float64) ** -1.1).astype(np.float32)   # a few large scores saturate
    comp, _ = _comp(n=n, eta=0.2, seed=3, tau=tau)
    assert comp.rule == "water" and comp.m_star > 0
    free = np.flatnonzero(~pc.forced_mask(n, 2, 4))
    saturated = sum(comp.r[i] == 1.0 for i in free)
    assert saturated == comp.m_star
    for i in free:
        assert pc.departing_probability(comp, float(tau[i])) == comp.r[i]


def test_departing_draw_frequency():
    """Over 4000 seeds the departing token is kept with frequency inside the 99.9%
    Clopper-Pearson interval of its r."""
    tau = np.random.default_rng(11).random(40).astype(np.float32)
    tau[40 - 4] = 0.3                                  # the token that leaves first
    hits, trials, r_t = 0, 4000, None
    for seed in range(trials):
        comp = pc.compress_head(tau, 2, 4, 0.3, 0, 0, 0, seed)
        new = pc.append_token(comp, 0.5, 2, 4, 0, 0, 0, seed)
        r_t = new.r[36]
        hits += int(new.resident[36])
    assert 0.0 < r_t < 1.0
    lo = stats.beta.ppf(0.0005, hits, trials - hits + 1) if hits else 0.0
    hi = stats.beta.ppf(0.9995, hits + 1, trials - hits) if hits < trials else 1.0
    assert lo <= r_t <= hi, (hits, r_t, lo, hi)


def test_the_other_branches_of_the_rule():
    tau = np.random.default_rng(2).random(32).astype(np.float32)
    tau[32 - 4] = 0.7
    # eta = 1: the budget covers every token, so a departing token stays
    comp = pc.compress_head(tau, 2, 4, 1.0, 0, 0, 0, 0)
    assert comp.rule == "all"
    new = pc.append_token(comp, 0.1, 2, 4, 0, 0, 0, 0)
    assert new.r[28] == 1.0 and new.resident[28]
    # budget exactly the forced tokens: no mass left for the others
    comp = pc.compress_head(tau, 2, 4, 6 / 32, 0, 0, 0, 0)
    assert comp.rule == "none"
    new = pc.append_token(comp, 0.1, 2, 4, 0, 0, 0, 0)
    assert new.r[28] == 0.0 and not new.resident[28]
    # tau = 0 under a water level: r = 0, never drawn, stays out of the sample
    tau0 = tau.copy()
    tau0[28] = 0.0
    comp = pc.compress_head(tau0, 2, 4, 0.3, 0, 0, 0, 0)
    assert comp.rule == "water"
    new = pc.append_token(comp, 0.1, 2, 4, 0, 0, 0, 0)
    assert new.r[28] == 0.0 and not new.resident[28]


def test_sink_tokens_never_leave():
    tau = np.full(6, 0.5, dtype=np.float32)
    comp = pc.compress_head(tau, 4, 4, 1.0, 0, 0, 0, 0)   # every token forced
    new = pc.append_token(comp, 0.5, 4, 4, 0, 0, 0, 0)    # t = 2 is a sink token
    assert np.all(new.r == 1.0) and np.all(new.resident)


def test_without_local_window_the_new_token_is_sampled():
    tau = np.random.default_rng(4).random(50).astype(np.float32)
    comp = pc.compress_head(tau, 2, 0, 0.25, 0, 0, 0, 9)
    new = pc.append_token(comp, 0.4, 2, 0, 0, 0, 0, 9)
    assert new.r[50] == pc.departing_probability(comp, 0.4)
    assert 0.0 < new.r[50] < 1.0
    assert np.array_equal(new.r[:50], comp.r)


@pytest.mark.parametrize("steps", [1, 5])
def test_grown_state_decodes_to_exact_attention_when_everything_is_fetched(steps):
    """eps tiny: every L token is fetched, so the estimator is exact attention over all
    n + steps tokens, including the appended ones (torch-free fp64 softmax reference)."""
    rng = np.random.default_rng(8)
    n, d, hkv, group = 96, 128, 2, 2
    tau = rng.random((hkv, n + steps)).astype(np.float32)
    K = rng.standard_normal((hkv, n + steps, d))
    V = rng.standard_normal((hkv, n + steps, d))
    q = rng.standard_normal((hkv * group, d))
    comp = oapi.compress_sequence(tau[:, :n], 2, 8, 0.25, 0, 0, 1)
    for s in range(steps):
        comp = oapi.append_sequence(comp, tau[:, n + s], 2, 8, 0, 0, 1)
    assert all(len(c.r) == n + steps for c in comp)
    out = oapi.decode_sequence(K, V, comp, q, group, 1.0, 1e-12, 0.05)
    for h in range(hkv * group):
        g = h // group
        s_ = K[g] @ q[h] / np.sqrt(d)
        w = np.exp(s_ - s_.max())
        o = (w[:, None] * V[g]).sum(0) / w.sum()
        assert np.allclose(out["o"][h], o, rtol=1e-10, atol=1e-12)
