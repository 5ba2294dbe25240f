"""KVFetch decode step: sketch weights, bounded shrinkage estimator, Bernstein
certificate, fetch ordering and refinement.  Test infrastructure for the oracle
only; float64 throughout.

Follows the picx.dev summary page, section "Methodology":
  * Definition 2 / eq. (5): D_hat = sum_H w_i + sum_L Z_i lambda_i w_i / r_i with
    lambda_i = clip_[r_i, 1](beta r_i / (w_i (1 - r_i))),
    clip_[r,1](x) = min{1, max{r, x}} and beta = sum_L w_i (1 - lambda_i);
  * Theorem 1 / eq. (6): the MSE that this estimator minimises;
  * Lemma 1 / eq. (7): eps_hat(L) = [beta(L) + b l/3 + sqrt((b l/3)^2 + 2 V l)] / D
    with l = log(2/delta), beta(L) = sum_L w_i (1 - lambda_i),
    V(L) = sum_L lambda_i^2 w_i^2 (1 - r_i) / r_i,
    b(L) = max_L lambda_i w_i max(r_i, 1 - r_i) / r_i;
  * subsection "KVFETCH": step 1 weights from the sketch, step 2 no fetch iff
    eps_hat(L) < eps, step 3 order by g_i = eps_hat(L) - eps_hat(L minus {i})
    (eq. 9), step 4 k* = min{k : eps_hat(L_g[k:]) < eps} (eq. 10), step 5 fetch
    L minus L' with L' = L_g[k*:] and refine;
  * the page's "Theoretical Foundation": the numerator N and the denominator D of
    attention are estimated and combined, o = N_hat / D_hat.

Readings where the page is silent or garbled (each listed in the design notes):
  * beta in the clip is the self-consistent value: the oracle solves
    B = sum_L w_i (1 - clip(kappa B r_i / (w_i (1 - r_i)))) exactly (a unique root;
    the right side is non-increasing in B).  kappa = 1 is Definition 2 as
    printed; kappa = inf gives lambda = 1 (Horvitz-Thompson), kappa = 0 gives
    lambda = r.
  * lambda, the certificate and g use the sketch weights w_hat (KVFetch step 1);
    the estimator uses weights from the true keys.  With the exact sketch (the
    sketch is the keys) the two coincide.  D in eq. (7) is sum over all n tokens
    of the sketch weights.
  * eq. (9) keeps lambda frozen at its value for the full L; removing token i
    removes its own terms, and b(L minus {i}) is the largest b of the others.
  * GQA: each query head makes its own decision; the fetched set of a KV head is
    the union over its query heads, and every head of the group treats all of it
    as exact.  Tokens fetched that are already resident cost no transfer.
  * ties in g are broken by token index, ascending.
  * log is the natural logarithm; scores are q.k / sqrt(d), shifted by the
    largest sketch score m_hat.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------- step 1
def sketch_weights(q: np.ndarray, K_sketch: np.ndarray):
    """KVFetch step 1: s_i = q.k_i / sqrt(d) over all n tokens, m_hat = max s,
    w_hat_i = exp(s_i - m_hat), D = sum_i w_hat_i.  Returns (w_hat, m_hat, D)."""
    q = np.asarray(q, dtype=np.float64)
    Ks = np.asarray(K_sketch, dtype=np.float64)
    s = (Ks @ q) / math.sqrt(q.shape[0])
    m_hat = float(np.max(s))
    w = np.exp(s - m_hat)
    return w, m_hat, float(np.sum(w))


# ----------------------------------------------------------------------------- lambda
def clip_lambda(w, r, B, kappa):
    """lambda_i = clip_[r_i, 1](kappa B r_i / (w_i (1 - r_i))) (Definition 2),
    with the conventions r_i = 0 -> lambda_i = 0 (never drawn), w_i = 0 ->
    lambda_i = 1, kappa = inf -> lambda_i = 1 on r_i > 0."""
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    lam = np.ones_like(w)
    reg = (r > 0.0) & (w > 0.0)
    if math.isinf(kappa):
        lam[reg] = 1.0
    else:
        x = (kappa * B * r[reg]) / (w[reg] * (1.0 - r[reg]))
        lam[reg] = np.minimum(1.0, np.maximum(r[reg], x))
    lam[r == 0.0] = 0.0
    return lam


def bias_of(w, r, B, kappa):
    """f(B) = sum_L w_i (1 - lambda_i(B)), the right side of the beta equation."""
    return float(np.sum(np.asarray(w, np.float64) * (1.0 - clip_lambda(w, r, B, kappa))))


def solve_beta(w, r, kappa):
    """The self-consistent beta of Definition 2: the root of B = f(B).

    f is continuous, piecewise linear and non-increasing in B, so B - f(B) is
    strictly increasing with one root in [0, f(0)].  Per token, with
    a_i = w_i (1 - r_i) / kappa and t_i = a_i / r_i: the term w_i (1 - lambda_i(B))
    equals w_i (1 - r_i) for B <= a_i, w_i - kappa B r_i / (1 - r_i) between, and 0
    for B >= t_i.  The root is found exactly: locate the breakpoint segment on
    which B - f(B) changes sign (binary search, B - f evaluated directly), then
    solve the linear equation B = C0 - C1 B of that segment.
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    k0 = float(np.sum(w[r == 0.0]))
    reg = (r > 0.0) & (w > 0.0)
    if math.isinf(kappa):
        return k0
    wr, rr = w[reg], r[reg]
    if kappa == 0.0:
        return k0 + float(np.sum(wr * (1.0 - rr)))
    a = wr * (1.0 - rr) / kappa
    t = a / rr
    slope = kappa * rr / (1.0 - rr)

    def segment(B):
        low = B <= a
        one = B >= t
        mid = ~low & ~one
        c0 = k0 + float(np.sum(wr[low] * (1.0 - rr[low]))) + float(np.sum(wr[mid]))
        c1 = float(np.sum(slope[mid]))
        return c0, c1

    def h(B):
        c0, c1 = segment(B)
        return B * (1.0 + c1) - c0

    bps = np.unique(np.concatenate([a, t]))
    bps = bps[bps > 0.0]
    lo, hi = -1, bps.size          # invariant: h(bps[lo]) <= 0 < h(bps[hi]) (virtual ends)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if h(float(bps[mid])) <= 0.0:
            lo = mid
        else:
            hi = mid
    left = float(bps[lo]) if lo >= 0 else 0.0
    right = float(bps[hi]) if hi < bps.size else math.inf
    inside = 0.5 * (left + right) if math.isfinite(right) else 2.0 * left + 1.0
    c0, c1 = segment(inside)
    return c0 / (1.0 + c1)


def solve_beta_bisect(w, r, kappa, iters=200):
    """Cross-check of solve_beta: plain bisection on B - f(B) over [0, f(0)]."""
    lo, hi = 0.0, bias_of(w, r, 0.0, kappa)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mid - bias_of(w, r, mid, kappa) <= 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# ----------------------------------------------------------------------------- certificate
def token_terms(w, r, lam):
    """Per-token pieces of eq. (7): beta_i = w_i (1 - lambda_i),
    V_i = lambda_i^2 w_i^2 (1 - r_i) / r_i, b_i = lambda_i w_i max(r_i, 1 - r_i) / r_i
    (V_i = b_i = 0 when r_i = 0: such a token is never drawn, so it has no variance)."""
    w = np.asarray(w, np.float64)
    r = np.asarray(r, np.float64)
    beta = w * (1.0 - lam)
    V = np.zeros_like(w)
    b = np.zeros_like(w)
    p = r > 0.0
    V[p] = lam[p] * lam[p] * w[p] * w[p] * (1.0 - r[p]) / r[p]
    b[p] = lam[p] * w[p] * np.maximum(r[p], 1.0 - r[p]) / r[p]
    return beta, V, b


def bernstein_E(beta, V, b, l):
    """Numerator of eq. (7): beta + b l/3 + sqrt((b l/3)^2 + 2 V l)."""
    t = b * l / 3.0
    return beta + t + math.sqrt(t * t + 2.0 * V * l)


def log_term(delta):
    """l_delta = log(2/delta), natural log (Lemma 1)."""
    return math.log(2.0 / delta)


def eps_hat(beta_i, V_i, b_i, D, l):
    """eps_hat over a token set given its per-token terms (empty set -> 0)."""
    if len(beta_i) == 0:
        return 0.0
    return bernstein_E(float(np.sum(beta_i)), float(np.sum(V_i)), float(np.max(b_i)), l) / D


def top2(b):
    """Largest and second-largest value of the multiset b (0 where absent)."""
    if b.size == 0:
        return 0.0, 0.0
    if b.size == 1:
        return float(b[0]), 0.0
    part = np.partition(b, b.size - 2)
    return float(part[-1]), float(part[-2])


def fetch_priority(beta_i, V_i, b_i, D, l):
    """g_i = eps_hat(L) - eps_hat(L minus {i}) (eq. 9) with lambda frozen.

    With b' = b(L minus {i}) (the runner-up if i holds the maximum, else the
    maximum), t = b l/3 and t' = b' l/3, X = t^2 + 2 V l, Y = t'^2 + 2 (V - V_i) l:
    D g_i = beta_i + (t - t') + (sqrt X - sqrt Y).  The square-root difference is
    evaluated as (X - Y) / (sqrt X + sqrt Y) with X - Y = (t - t')(t + t') + 2 V_i l,
    the same number without the cancellation."""
    V = float(np.sum(V_i))
    b1, b2 = top2(b_i)
    bm = np.where(b_i == b1, b2, b1)
    t1 = b1 * l / 3.0
    tm = bm * l / 3.0
    X = t1 * t1 + 2.0 * V * l
    Y = tm * tm + 2.0 * (V - V_i) * l
    dX = (t1 - tm) * (t1 + tm) + 2.0 * V_i * l
    den = math.sqrt(X) + np.sqrt(Y)
    frac = np.where(den > 0.0, dX / np.where(den > 0.0, den, 1.0), 0.0)
    gD = beta_i + (t1 - tm) + frac
    return gD / D


def select_fetch(tokens, beta_i, V_i, b_i, D, l, eps):
    """KVFetch steps 3-4: order L by (g desc, token asc) and return
    (F_h, k*, g) where F_h is the first k* tokens and k* is the smallest k with
    eps_hat(L_g[k:]) < eps (eq. 10); the suffix sums are the sums over L_g[k:]."""
    g = fetch_priority(beta_i, V_i, b_i, D, l)
    order = np.lexsort((tokens, -g))
    sb = beta_i[order][::-1].cumsum()[::-1]
    sV = V_i[order][::-1].cumsum()[::-1]
    smax = np.maximum.accumulate(b_i[order][::-1])[::-1]
    t = smax * l / 3.0
    E = np.append(sb + t + np.sqrt(t * t + 2.0 * sV * l), 0.0)     # E(L_g[k:]), k = 0..|L|
    kstar = int(np.flatnonzero(E / D < eps)[0])
    return np.sort(tokens[order[:kstar]]), kstar, g


# ----------------------------------------------------------------------------- one step
@dataclass
class HeadDecision:
    m_hat: float
    D: float
    beta_star: float
    eps_hat: float
    certified: bool
    kstar: int
    fetch: np.ndarray      # this head's F_h (ascending)
    lam: np.ndarray        # [n] lambda (0 outside L... 1 on H)
    terms: tuple           # (beta_i, V_i, b_i) over L, in token order
    L: np.ndarray          # token ids of L (ascending)


def decide_head(q, K_sketch, r, kappa, eps, delta) -> HeadDecision:
    """KVFetch steps 1-4 for one query head."""
    w, m_hat, D = sketch_weights(q, K_sketch)
    L = np.flatnonzero(r < 1.0)
    wL, rL = w[L], r[L]
    B = solve_beta(wL, rL, kappa)
    lamL = clip_lambda(wL, rL, B, kappa)
    beta_i, V_i, b_i = token_terms(wL, rL, lamL)
    l = log_term(delta)
    e = eps_hat(beta_i, V_i, b_i, D, l)
    lam = np.ones(r.shape[0])
    lam[L] = lamL
    if e < eps:
        return HeadDecision(m_hat, D, B, e, True, 0, np.zeros(0, np.int64), lam,
                            (beta_i, V_i, b_i), L)
    F, kstar, _ = select_fetch(L, beta_i, V_i, b_i, D, l, eps)
    return HeadDecision(m_hat, D, B, e, False, kstar, F, lam, (beta_i, V_i, b_i), L)


def estimate(q, K, Vv, r, resident, fetched, lam, m_hat):
    """Eq. (5) for D and its numerator analogue N, with the fetched tokens exact:
    D_hat = sum_{H u F} w_i + sum_{S \\ F} lambda_i w_i / r_i, N_hat likewise with
    w_i v_i; w_i from the true keys, shifted by m_hat.  Returns (N_hat, D_hat)."""
    q = np.asarray(q, np.float64)
    n = r.shape[0]
    coef = np.zeros(n)
    exact = (r >= 1.0)
    exact[fetched] = True
    sampled = resident & ~exact
    coef[exact] = 1.0
    coef[sampled] = lam[sampled] / r[sampled]
    use = np.flatnonzero(coef > 0.0)
    Ku = np.asarray(K[use], np.float64)
    Vu = np.asarray(Vv[use], np.float64)
    w = np.exp((Ku @ q) / math.sqrt(q.shape[0]) - m_hat)
    cw = coef[use] * w
    return cw @ Vu, float(np.sum(cw))


def decode_kv_head(qs, K, Vv, r, resident, kappa, eps, delta, K_sketch=None, resolved=None):
    """One KV head, its G query rows: decisions, union F, estimator, refinement.
    resolved: None for the frozen reading of eq. (9)-(10); "scan" or "bisect" for the
    re-solved reading (decide_head_resolved, k* by the scan or by bisection).

    Returns a dict of per-row lists and the KV-head fetch set."""
    Ks = K if K_sketch is None else K_sketch
    if resolved is None:
        decs = [decide_head(q, Ks, r, kappa, eps, delta) for q in qs]
    else:
        decs = [decide_head_resolved(q, Ks, r, kappa, eps, delta, bisect=resolved == "bisect")
                for q in qs]
    F = np.unique(np.concatenate([d.fetch for d in decs])) if decs else np.zeros(0, np.int64)
    F = F.astype(np.int64)
    inF = np.zeros(r.shape[0], dtype=bool)
    inF[F] = True
    l = log_term(delta)
    out = {"m_hat": [], "D": [], "beta_star": [], "eps_hat": [], "certified": [], "kstar": [],
           "eps_after": [], "n_hat": [], "d_hat": [], "o": [], "lse": []}
    for q, d in zip(qs, decs):
        keep = ~inF[d.L]
        bi, Vi, b_i = d.terms
        e_after = eps_hat(bi[keep], Vi[keep], b_i[keep], d.D, l)
        N, Dh = estimate(q, K, Vv, r, resident, F, d.lam, d.m_hat)
        out["m_hat"].append(d.m_hat)
        out["D"].append(d.D)
        out["beta_star"].append(d.beta_star)
        out["eps_hat"].append(d.eps_hat)
        out["certified"].append(d.certified)
        out["kstar"].append(d.kstar)
        out["eps_after"].append(e_after)
        out["n_hat"].append(N)
        out["d_hat"].append(Dh)
        out["o"].append(N / Dh)
        out["lse"].append(d.m_hat + math.log(Dh))
    out = {k: np.asarray(v) for k, v in out.items()}
    out["fetch"] = F
    out["h2d"] = F[~resident[F]]
    return out


# ------------------------------------------------------------ re-solved lambda (variant)
# Eq. (9) writes eps_hat(L minus {i}) without saying whether lambda follows the set.  The
# decision path above freezes lambda at its value for the full L (the frozen reading, the one the
# library implements).  The variant below re-solves the bias of Definition 2, and so
# lambda, on every candidate set of step 4 (the re-solved reading).  Taken here for it:
#   * the order of step 3 is the frozen one (g_i of eq. 9): re-solving for every
#     single removal would cost |L| solves per row for an ordering only;
#   * the cut of step 4 evaluates each candidate L_g[k:] with lambda solved on that set
#     alone, and k* is the least such k, found by a scan from k = 0 (with re-solved lambda
#     eps_hat need not fall monotonically in k, so no bisection);
#   * the kept set L' = L_g[k*:] keeps the lambda solved on it.
# Lemma 1 still certifies the result: lambda(L') depends on the sketch weights and r, not
# on the draws Z.  Parity unpinned against the pages (they give no example); pinned by
# tests/test_oracle_resolved.py (reductions to the frozen reading where lambda ignores the
# bias, brute force with an independent bisection solve on small sets).
def eps_hat_resolved(w, r, kappa, D, l):
    """eps_hat of one token set with the bias and lambda solved on that set alone."""
    w = np.asarray(w, np.float64)
    r = np.asarray(r, np.float64)
    if w.size == 0:
        return 0.0
    B = solve_beta(w, r, kappa)
    lam = clip_lambda(w, r, B, kappa)
    return eps_hat(*token_terms(w, r, lam), D, l)


def select_fetch_resolved(tokens, w, r, kappa, beta_i, V_i, b_i, D, l, eps):
    """Steps 3-4, re-solved reading: (F_h, k*, g) with the order of eq. (9) and k* the least
    k with eps_hat_resolved(L_g[k:]) < eps."""
    g = fetch_priority(beta_i, V_i, b_i, D, l)
    order = np.lexsort((tokens, -g))
    for k in range(order.size + 1):
        rest = order[k:]
        if eps_hat_resolved(w[rest], r[rest], kappa, D, l) < eps:
            return np.sort(tokens[order[:k]]), k, g
    raise AssertionError("eps_hat of the empty set is 0, below any eps > 0")


def select_fetch_resolved_bisect(tokens, w, r, kappa, beta_i, V_i, b_i, D, l, eps):
    """Steps 3-4 of the re-solved reading with k* found by bisection over k.

    eps_hat of L_g[k:] with the bias solved on that set is non-increasing in k: for
    S' inside S the bias function of S' lies below that of S at every B, so its fixed
    point is no larger; lambda_i, V_i and b_i are non-decreasing in B, so V(S') <= V(S)
    and b(S') <= b(S); and eq. (7)'s numerator grows with each of beta, V and b.  The
    least k with eps_hat < eps is therefore the boundary of a monotone predicate, and
    bisection over k in [0, |L|] (the empty set has eps_hat = 0) finds the scan's k*
    with about log2 |L| solves instead of up to |L|.  Rounding can break monotonicity
    only between candidates whose eps_hat agree to rounding, so the two differ only when
    eps_hat at the cut is within rounding of eps."""
    g = fetch_priority(beta_i, V_i, b_i, D, l)
    order = np.lexsort((tokens, -g))

    def certifies(k):
        rest = order[k:]
        return eps_hat_resolved(w[rest], r[rest], kappa, D, l) < eps

    lo, hi = 0, order.size                 # certifies(hi) holds: the empty set
    if certifies(0):
        hi = 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if certifies(mid):
            hi = mid
        else:
            lo = mid
    return np.sort(tokens[order[:hi]]), hi, g


def decide_head_resolved(q, K_sketch, r, kappa, eps, delta, bisect=False) -> HeadDecision:
    """KVFetch steps 1-4 for one query head, re-solved reading.  Certification (k* = 0) is
    the frozen reading's test; a fetching row gets lambda solved on its kept set L', and its
    beta_star, terms and L fields then describe L' (the set its certificate covers)."""
    w, m_hat, D = sketch_weights(q, K_sketch)
    L = np.flatnonzero(r < 1.0)
    wL, rL = w[L], r[L]
    B = solve_beta(wL, rL, kappa)
    lamL = clip_lambda(wL, rL, B, kappa)
    beta_i, V_i, b_i = token_terms(wL, rL, lamL)
    l = log_term(delta)
    e = eps_hat(beta_i, V_i, b_i, D, l)
    lam = np.ones(r.shape[0])
    lam[L] = lamL
    if e < eps:
        return HeadDecision(m_hat, D, B, e, True, 0, np.zeros(0, np.int64), lam,
                            (beta_i, V_i, b_i), L)
    select = select_fetch_resolved_bisect if bisect else select_fetch_resolved
    F, kstar, _ = select(L, wL, rL, kappa, beta_i, V_i, b_i, D, l, eps)
    keep = np.ones(L.size, dtype=bool)
    keep[np.searchsorted(L, F)] = False
    Bk = solve_beta(wL[keep], rL[keep], kappa)
    lam[L[keep]] = clip_lambda(wL[keep], rL[keep], Bk, kappa)
    kept_terms = token_terms(wL[keep], rL[keep], lam[L[keep]])
    return HeadDecision(m_hat, D, Bk, e, False, kstar, F, lam, kept_terms, L[keep])
