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


@pytest.mark.parametrize("seed", range(8))
def test_bisection_finds_the_scans_cut(seed):
    """k* by bisection over k equals the scan's least k (eps_hat of the re-solved reading
    is non-increasing in k), on rows whose candidates all stay clear of eps."""
    q, K, r = _row(200 + seed, n=400)
    w, _, D = kf.sketch_weights(q, K)
    L = np.flatnonzero(r < 1.0)
    wL, rL = w[L], r[L]
    l = kf.log_term(0.05)
    B = kf.solve_beta(wL, rL, 1.0)
    bi, Vi, b_i = kf.token_terms(wL, rL, kf.clip_lambda(wL, rL, B, 1.0))
    eps = 0.25 * kf.eps_hat(bi, Vi, b_i, D, l)
    F1, k1, g = kf.select_fetch_resolved(L, wL, rL, 1.0, bi, Vi, b_i, D, l, eps)
    F2, k2, _ = kf.select_fetch_resolved_bisect(L, wL, rL, 1.0, bi, Vi, b_i, D, l, eps)
    assert k1 > 0 and k1 == k2 and np.array_equal(F1, F2)


@pytest.mark.parametrize("seed", range(4))
def test_resolved_eps_hat_is_monotone_in_k(seed):
    """The property the bisection rests on, checked at every k of a 300-token row."""
    q, K, r = _row(300 + seed)
    w, _, D = kf.sketch_weights(q, K)
    L = np.flatnonzero(r < 1.0)
    wL, rL = w[L], r[L]
    l = kf.log_term(0.05)
    B = kf.solve_beta(wL, rL, 1.0)
    terms = kf.token_terms(wL, rL, kf.clip_lambda(wL, rL, B, 1.0))
    order = np.lexsort((L, -kf.fetch_priority(*terms, D, l)))
    vals = [kf.eps_hat_resolved(wL[order[k:]], rL[order[k:]], 1.0, D, l) for k in range(L.size + 1)]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(vals, vals[1:]))
    assert vals[-1] == 0.0


def test_resolved_decode_of_a_kv_head_certifies_every_row():
    """decode_kv_head with the re-solved reading: every row ends with eps_hat(L' minus F)
    below eps, the union F is at most the frozen reading's here, and both forms of the
    cut agree."""
    q, K, r = _row(400)
    rng = np.random.default_rng(1)
    V = rng.standard_normal(K.shape)
    qs = [q, q * 1.2, -q]
    resident = r >= 1.0
    a = kf.decode_kv_head(qs, K, V, r, resident, 1.0, 0.05, 0.05, resolved="scan")
    b = kf.decode_kv_head(qs, K, V, r, resident, 1.0, 0.05, 0.05, resolved="bisect")
    fz = kf.decode_kv_head(qs, K, V, r, resident, 1.0, 0.05, 0.05)
    assert np.array_equal(a["fetch"], b["fetch"]) and np.array_equal(a["kstar"], b["kstar"])
    assert np.all(a["eps_after"] < 0.05)
    assert a["fetch"].size <= fz["fetch"].size
