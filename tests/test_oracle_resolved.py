"""Pins of the oracle's re-solved reading of eq. (9)-(10) (oracle/kvfetch.py: lambda
re-solved on each candidate set of the cut).  The pages print no worked example, so the
pins are reductions and brute force: where lambda does not depend on the bias (kappa = inf
gives lambda = 1, kappa = 0 gives lambda = r) it must fetch exactly what the frozen reading
fetches; on small sets the least k found by the scan must match a search that solves the
bias by plain bisection and sums eq. (7) term by term; the bias it keeps is the fixed point
on its kept set, and the kept set certifies."""
import math

import numpy as np
import pytest

from oracle import kvfetch as kf


def _row(seed, n=300, d=128, scale=0.35):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d))
    q = rng.standard_normal(d) * scale
    r = rng.random(n) * 0.4
    r[:4] = 1.0
    r[-16:] = 1.0
    r[rng.choice(n, 8, replace=False)] = 0.0
    return q, K, r


@pytest.mark.parametrize("kappa", [math.inf, 0.0])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_reduces_to_frozen_lambda_when_lambda_ignores_the_bias(kappa, seed):
    q, K, r = _row(seed)
    a = kf.decide_head(q, K, r, kappa, 0.05, 0.05)
    b = kf.decide_head_resolved(q, K, r, kappa, 0.05, 0.05)
    assert not a.certified and a.kstar > 0
    assert b.kstar == a.kstar
    assert np.array_equal(b.fetch, a.fetch)


@pytest.mark.parametrize("seed", [3, 4])
def test_certification_is_the_frozen_test(seed):
    q, K, _ = _row(seed, scale=0.02)
    rng = np.random.default_rng(seed)
    r = 0.6 + 0.35 * rng.random(K.shape[0])    # flat scores, large r: eps_hat near 0.09
    r[:4] = 1.0
    r[-16:] = 1.0
    a = kf.decide_head(q, K, r, 1.0, 0.2, 0.05)
    b = kf.decide_head_resolved(q, K, r, 1.0, 0.2, 0.05)
    assert a.certified and b.certified and b.kstar == 0 and b.fetch.size == 0
    assert b.eps_hat == a.eps_hat


def _bias_bisect(w, r, kappa):
    """Root of B = sum w (1 - clip_[r,1](kappa B r / (w (1 - r)))) by bisection, written
    out per token (r = 0: lambda = 0)."""
    def f(B):
        tot = 0.0
        for wi, ri in zip(w, r):
            if ri == 0.0:
                lam = 0.0
            else:
                lam = min(1.0, max(ri, kappa * B * ri / (wi * (1.0 - ri))))
            tot += wi * (1.0 - lam)
        return tot
    lo, hi = 0.0, f(0.0)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid - f(mid) > 0.0:
            hi = mid
        else:
            lo = mid
    return 0.5 * (lo + hi)


def _eps_brute(w, r, kappa, D, l):
    if len(w) == 0:
        return 0.0
    B = _bias_bisect(w, r, kappa)
    sb = sv = mb = 0.0
    for wi, ri in zip(w, r):
        lam = 0.0 if ri == 0.0 else min(1.0, max(ri, kappa * B * ri / (wi * (1.0 - ri))))
        sb += wi * (1.0 - lam)
        if ri > 0.0:
            sv += lam * lam * wi * wi * (1.0 - ri) / ri
            mb = max(mb, lam * wi * max(ri, 1.0 - ri) / ri)
    t = mb * l / 3.0
    return (sb + t + math.sqrt(t * t + 2.0 * sv * l)) / D


@pytest.mark.parametrize("seed", range(12))
def test_least_k_matches_brute_force_on_small_sets(seed):
    rng = np.random.default_rng(100 + seed)
    nL = int(rng.integers(3, 11))
    tokens = np.arange(nL, dtype=np.int64) * 3 + 5
    w = np.exp(rng.standard_normal(nL) * 1.5)
    r = rng.random(nL) * 0.9 + 0.02
    if seed % 3 == 0:
        r[0] = 0.0
    D = float(np.sum(w)) + float(rng.random() * 4.0 + 0.5)
    l = kf.log_term(0.05)
    kappa = 1.0
    B = kf.solve_beta(w, r, kappa)
    lam = kf.clip_lambda(w, r, B, kappa)
    bi, Vi, b_i = kf.token_terms(w, r, lam)
    eps = 0.5 * kf.eps_hat(bi, Vi, b_i, D, l)
    F, kstar, g = kf.select_fetch_resolved(tokens, w, r, kappa, bi, Vi, b_i, D, l, eps)
    order = np.lexsort((tokens, -g))
    vals = [_eps_brute(w[order[k:]], r[order[k:]], kappa, D, l) for k in range(nL + 1)]
    if any(abs(v - eps) <= 1e-9 * eps for v in vals):
        pytest.skip("a candidate lies within rounding of eps")
    k_brute = next(k for k, v in enumerate(vals) if v < eps)
    assert kstar == k_brute
    assert np.array_equal(F, np.sort(tokens[order[:k_brute]]))


@pytest.mark.parametrize("seed", [5, 6])
def test_kept_bias_is_the_fixed_point_and_certifies(seed):
    q, K, r = _row(seed)
    d = kf.decide_head_resolved(q, K, r, 1.0, 0.05, 0.05)
    assert not d.certified and d.kstar > 0
    w, _, D = kf.sketch_weights(q, K)
    wk, rk = w[d.L], r[d.L]
    assert abs(d.beta_star - kf.bias_of(wk, rk, d.beta_star, 1.0)) <= 1e-12 * max(1.0, d.beta_star)
    assert kf.eps_hat(*d.terms, D, kf.log_term(0.05)) < 0.05
    assert np.all(d.lam[d.fetch] == kf.decide_head(q, K, r, 1.0, 0.05, 0.05).lam[d.fetch])
