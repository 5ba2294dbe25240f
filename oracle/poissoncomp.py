"""PoissonComp: inclusion probabilities by water-filling and the Poisson sample.
Test infrastructure for the oracle only.

Follows the picx.dev summary page, section "Methodology", subsection
"POISSONCOMP: Stochastic KV Cache Compression":
  * eq. (3): r_i = min{1, c*tau_i}, with c chosen so that sum_i min(1, c*tau_i) = eta*n;
  * H = tokens kept with probability 1 (sink and local tokens among them),
    L = tokens with r_i < 1;
  * S = {i in L : Z_i = 1}, Z_i ~ Bernoulli(r_i), all independent.

Readings where the page is silent (each also listed in the design notes):
  * eta is a fraction of n (the page writes both "a budget of eta tokens" and
    sum = eta*n); the budget is fl(eta*n) tokens and the forced sink/local tokens
    count toward it: the remaining probability mass fl(eta*n) - |H_forced| is
    water-filled over the other tokens.
  * Exact arithmetic for c: tau (float32) is turned into the integer
    Q_i = ceil(tau_i * 2^40) and every sum of Q is an exact integer, so r is a
    deterministic function of the inputs.  The water level for "the first m
    tokens saturated" is c_m = fl(fl(B_rem - m) / fl(S_m)) with
    S_m = sum of Q over ranks >= m (ranks by Q descending, index ascending);
    m* is the smallest m with B_rem - m > 0, S_m > 0 and fl(c_m * Q_(m)) < 1.
  * tau_i = 0 gives Q_i = 0 and r_i = 0: such a token is never drawn.  It stays
    in L for the certificate (its weight is pure bias).
  * Z_i = [u_i < r_i] with u_i the 53-bit Philox uniform of counter
    (i, kv_head, layer, stream) under key (seed mod 2^32, seed >> 32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import philox

Q_BITS = 40


class BudgetError(ValueError):
    """eta*n is smaller than the number of forced sink + local tokens."""


@dataclass
class Compressed:
    r: np.ndarray          # [n] float64, 1 on H
    resident: np.ndarray   # [n] bool, H union S
    piv_idx: np.ndarray    # ascending int64 token ids of H union S
    m_star: int            # saturated non-forced tokens (-1: none qualified)
    c: float               # water level (0 when unused)
    rule: str = "water"    # how the prefill set r on non-forced tokens (see level_rule)
    tau: np.ndarray = None # [n] float32 scores (kept for tokens leaving the local window)


def forced_mask(n: int, n_sink: int, n_local: int) -> np.ndarray:
    """Sink tokens 0..n_sink-1 and local tokens n-n_local..n-1 (always kept)."""
    m = np.zeros(n, dtype=bool)
    m[:min(n_sink, n)] = True
    if n_local > 0:
        m[max(0, n - n_local):] = True
    return m


def quantize(tau: np.ndarray) -> list:
    """Q_i = ceil(tau_i * 2^40) as exact Python integers (tau*2^40 is exact in fp64)."""
    t = np.asarray(tau, dtype=np.float32).astype(np.float64) * float(1 << Q_BITS)
    return [int(math.ceil(x)) for x in t]


def inclusion_probabilities(tau, n_sink, n_local, eta):
    """Water-filling of eq. (3).  Returns (r, m_star, c)."""
    tau = np.asarray(tau, dtype=np.float32)
    n = tau.shape[0]
    if not (0.0 < eta <= 1.0):
        raise ValueError("eta must lie in (0, 1]")
    if np.any(~(tau >= 0.0)) or np.any(tau > 1.0):
        raise ValueError("tau must lie in [0, 1]")
    forced = forced_mask(n, n_sink, n_local)
    r = np.zeros(n, dtype=np.float64)
    r[forced] = 1.0
    budget = float(eta) * float(n)
    b_rem = budget - float(int(forced.sum()))
    if b_rem < 0.0:
        raise BudgetError(f"eta*n = {budget} < {int(forced.sum())} forced tokens")
    free = np.flatnonzero(~forced)
    if free.size == 0 or b_rem == 0.0:
        return r, 0, 0.0
    if b_rem >= float(free.size):
        r[free] = 1.0
        return r, free.size, 0.0
    q = quantize(tau[free])
    # ranks: Q descending, token index ascending
    order = sorted(range(free.size), key=lambda j: (-q[j], free[j]))
    qs = [q[j] for j in order]
    suffix = [0] * (free.size + 1)
    for m in range(free.size - 1, -1, -1):
        suffix[m] = suffix[m + 1] + qs[m]
    m_star, c_star = -1, 0.0
    for m in range(free.size):
        rem = b_rem - float(m)
        if not (rem > 0.0) or suffix[m] <= 0:
            continue
        c_m = rem / float(suffix[m])
        if c_m * float(qs[m]) < 1.0:
            m_star, c_star = m, c_m
            break
    if m_star < 0:
        # every positive-score token saturates; the budget cannot be spent
        for j in range(free.size):
            r[free[j]] = 1.0 if q[j] > 0 else 0.0
        return r, -1, 0.0
    for rank, j in enumerate(order):
        r[free[j]] = 1.0 if rank < m_star else c_star * float(q[j])
    return r, m_star, c_star


def draw(r: np.ndarray, kv_head: int, layer: int, stream: int, seed: int) -> np.ndarray:
    """Poisson sample: Z_i = [u_i < r_i] for tokens of L with r_i > 0; returns the
    resident mask H union S."""
    r = np.asarray(r, dtype=np.float64)
    resident = r >= 1.0
    cand = np.flatnonzero((r < 1.0) & (r > 0.0))
    if cand.size:
        u = philox.uniform53(cand, kv_head, layer, stream, seed)
        resident[cand[u < r[cand]]] = True
    return resident


def level_rule(n, n_sink, n_local, eta, m_star):
    """Which branch of the water-filling set r on the non-forced tokens:
    "all" (the budget covers them all: r = 1), "none" (no budget left: r = 0),
    "saturated" (no water level qualified: r = 1 where tau > 0, else 0) or "water"
    (r = min(1, c Q) with the level c)."""
    forced = int(forced_mask(n, n_sink, n_local).sum())
    free = n - forced
    b_rem = float(eta) * float(n) - float(forced)
    if free == 0 or b_rem >= float(free):
        return "all"
    if b_rem == 0.0:
        return "none"
    return "saturated" if m_star < 0 else "water"


def compress_head(tau, n_sink, n_local, eta, kv_head, layer, stream, seed) -> Compressed:
    r, m_star, c = inclusion_probabilities(tau, n_sink, n_local, eta)
    resident = draw(r, kv_head, layer, stream, seed)
    return Compressed(r=r, resident=resident, piv_idx=np.flatnonzero(resident),
                      m_star=m_star, c=c, rule=level_rule(len(r), n_sink, n_local, eta, m_star),
                      tau=np.asarray(tau, dtype=np.float32).copy())


# ------------------------------------------------------------------ a growing cache
# The pages compress the cache once, at prefill, and say nothing about the tokens decode
# appends.  Reading taken here (parity unpinned against the pages; pinned by the
# properties in tests/test_oracle_append.py):
#   * the appended token n joins the local window: r_n = 1, resident;
#   * the token leaving the window, t = n - n_local, becomes an ordinary token unless it
#     is a sink token: it gets the prefill's rule with the prefill's water level,
#     r_t = min(1, fl(c Q_t)) (or 1 / 0 / 1-if-tau>0 for the "all" / "none" /
#     "saturated" branches), and if 0 < r_t < 1 it is drawn with the Philox counter
#     (t, kv_head, layer, stream) it would have had at prefill;
#   * without a local window (n_local = 0) the appended token itself is the one that
#     gets the rule and the draw;
#   * the level is not re-solved, so the resident budget grows by r_t per token.
def departing_probability(comp: Compressed, tau_t: float) -> float:
    """r of a token that leaves the forced set, under the prefill's rule."""
    q = quantize(np.array([tau_t], dtype=np.float32))[0]
    if comp.rule == "all":
        return 1.0
    if comp.rule == "none":
        return 0.0
    if comp.rule == "saturated":
        return 1.0 if q > 0 else 0.0
    x = comp.c * float(q)
    return 1.0 if x >= 1.0 else x


def append_token(comp: Compressed, tau_new: float, n_sink: int, n_local: int,
                 kv_head: int, layer: int, stream: int, seed: int) -> Compressed:
    """The compressed state of one KV head after token n = len(comp.r) is appended."""
    n = len(comp.r)
    r = np.concatenate([comp.r, [1.0]])
    resident = np.concatenate([comp.resident, [True]])
    tau = np.concatenate([comp.tau, np.array([tau_new], dtype=np.float32)])
    t = n - n_local                       # the token leaving the window (n itself when n_local = 0)
    if n_local >= 0 and n_sink <= t <= n:
        rt = departing_probability(comp, float(tau[t]))
        r[t] = rt
        if rt >= 1.0:
            resident[t] = True
        elif rt > 0.0:
            u = philox.uniform53(np.array([t]), kv_head, layer, stream, seed)
            resident[t] = bool(u[0] < rt)
        else:
            resident[t] = False
    return Compressed(r=r, resident=resident, piv_idx=np.flatnonzero(resident),
                      m_star=comp.m_star, c=comp.c, rule=comp.rule, tau=tau)
