"""Helpers for the GPU-vs-oracle parity tests: run the oracle on a workload and
compare with the library's results to the parity standard:

  * r, the resident mask and the pivot lists: bit-exact;
  * certified flags, k* and the fetch lists: exact, except for a row whose certificate
    statistic (eps_hat(L) against eps, or eps_hat(L_g[k:]) at the k* cut) lies within
    1e-6 relative of eps;
  * m_hat, D, beta*, eps_hat: float64 results of the same formulas in another summation
    order, compared at 1e-9 relative;
  * o, N_hat and D_hat (bf16 inputs, float32 accumulation): 2e-3 relative L2 per row;
    lse within 2e-3 absolute.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import api as oapi
from oracle import kvfetch as okf

NEAR = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu_library():
    """Skip without a GPU; otherwise load libverkv.so and require that it was built from
    the sources in this tree (the hash the build compiles in), so a stale library is
    never the one tested."""
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_decode_kvfetch_amd import build, verkv
    got = verkv.lib().verkv_source_hash().decode()
    want = build.source_hash()
    assert got == want, f"libverkv.so was built from other sources ({got[:12]} != {want[:12]}); rebuild it"


def oracle_compress(wl):
    """Per sequence: list over KV heads of poissoncomp.Compressed."""
    return [oapi.compress_sequence(s.tau, wl.n_sink, wl.n_local, wl.eta, wl.layer, b, wl.seed)
            for b, s in enumerate(wl.seqs)]


def oracle_step(wl, comp, step, kappa=None, eps=None, delta=None, sketch_of=None, resolved=None):
    """The oracle's step for every sequence; `sketch_of` maps a KV head's key rows to the
    sketch keys its weights come from (None: the keys themselves); `resolved` selects the
    re-solved reading of eqs. (9)-(10) ("scan" or "bisect"; None: lambda frozen)."""
    kappa = wl.kappa if kappa is None else kappa
    eps = wl.eps if eps is None else eps
    delta = wl.delta if delta is None else delta
    outs = []
    for b, s in enumerate(wl.seqs):
        Ks = None if sketch_of is None else np.stack([sketch_of(s.K[g]) for g in range(s.K.shape[0])])
        outs.append(oapi.decode_sequence(s.K, s.V, comp[b], wl.queries[step, b], wl.group,
                                         kappa, eps, delta, K_sketch=Ks, resolved=resolved))
    return outs


def cut_near_threshold_resolved(comp_bg, q, kappa, eps, delta, K, kstars):
    """Re-solved reading: True if eps_hat of L_g[k:] (bias solved on it) lies within NEAR
    of eps at any cut k the two sides found, or just before it."""
    w, _, D = okf.sketch_weights(q, K)
    r = comp_bg.r
    L = np.flatnonzero(r < 1.0)
    wL, rL = w[L], r[L]
    l = okf.log_term(delta)
    B = okf.solve_beta(wL, rL, kappa)
    terms = okf.token_terms(wL, rL, okf.clip_lambda(wL, rL, B, kappa))
    order = np.lexsort((L, -okf.fetch_priority(*terms, D, l)))
    for k0 in kstars:
        for k in (k0 - 1, k0):
            if 0 <= k <= L.size:
                v = okf.eps_hat_resolved(wL[order[k:]], rL[order[k:]], kappa, D, l)
                if abs(v - eps) <= NEAR * eps:
                    return True
    return False


def cut_near_threshold(wl, comp_bg, q, kappa, eps, delta, K):
    """True if this row's decision or its k* cut is within NEAR of eps (oracle view)."""
    d = okf.decide_head(q, K, comp_bg.r, kappa, eps, delta)
    if abs(d.eps_hat - eps) <= NEAR * eps:
        return True
    if d.certified:
        return False
    bi, Vi, b_i = d.terms
    l = okf.log_term(delta)
    g = okf.fetch_priority(bi, Vi, b_i, d.D, l)
    order = np.lexsort((d.L, -g))
    k = d.kstar
    vals = []
    for kk in (k - 1, k):
        if 0 <= kk <= d.L.size:
            sel = order[kk:]
            vals.append(okf.eps_hat(bi[sel], Vi[sel], b_i[sel], d.D, l))
    return any(abs(v - eps) <= NEAR * eps for v in vals)


def compare_state(sess, wl, ocomp):
    got = sess.state_numpy()
    u = 0
    for b, s in enumerate(wl.seqs):
        for g in range(wl.n_kv_heads):
            oc = ocomp[b][g]
            gs = got[u]
            assert np.array_equal(gs["r"].view(np.uint64), oc.r.view(np.uint64)), (b, g, "r")
            assert np.array_equal(gs["resident"], oc.resident), (b, g, "resident")
            assert gs["piv_count"] == oc.piv_idx.size, (b, g, "count")
            assert np.array_equal(gs["piv_idx"], oc.piv_idx), (b, g, "piv_idx")
            u += 1


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def compare_step(sess, wl, ocomp, oouts, step, kappa=None, eps=None, delta=None, tol=2e-3,
                 sketch_of=None, resolved=None):
    """Compare one step; returns a dict of summary numbers."""
    kappa = wl.kappa if kappa is None else kappa
    eps = wl.eps if eps is None else eps
    delta = wl.delta if delta is None else delta
    res = sess.results_numpy()
    hq = wl.n_q_heads
    G = wl.group
    worst = 0.0
    exempt_units = set()
    for b, s in enumerate(wl.seqs):
        oo = oouts[b]
        sl = slice(b * hq, (b + 1) * hq)
        np.testing.assert_allclose(res["m_hat"][sl], oo["m_hat"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["d_sketch"][sl], oo["D"], rtol=1e-9)
        if resolved is None:
            np.testing.assert_allclose(res["beta_star"][sl], oo["beta_star"], rtol=1e-9, atol=1e-300)
        np.testing.assert_allclose(res["eps_hat"][sl], oo["eps_hat"], rtol=1e-9, atol=1e-300)
        for h in range(hq):
            row = b * hq + h
            g = h // G
            near = None
            if bool(res["certified"][row]) != bool(oo["certified"][h]) or \
                    int(res["kstar"][row]) != int(oo["kstar"][h]):
                Kd = s.K[g] if sketch_of is None else sketch_of(s.K[g])
                if resolved is None:
                    near = cut_near_threshold(wl, ocomp[b][g], wl.queries[step, b, h], kappa, eps,
                                              delta, Kd)
                else:
                    near = cut_near_threshold_resolved(
                        ocomp[b][g], wl.queries[step, b, h], kappa, eps, delta, Kd,
                        (int(res["kstar"][row]), int(oo["kstar"][h])))
                assert near, (b, h, "decision", res["certified"][row], oo["certified"][h],
                              res["kstar"][row], oo["kstar"][h], res["eps_hat"][row])
                exempt_units.add((b, g))
        if resolved is not None:
            # the kept set's bias (the full L's for certified rows)
            for h in range(hq):
                if (b, h // G) not in exempt_units:
                    np.testing.assert_allclose(res["beta_star"][b * hq + h], oo["beta_star"][h],
                                               rtol=1e-9, atol=1e-300)
        for g in range(wl.n_kv_heads):
            u = b * wl.n_kv_heads + g
            if (b, g) in exempt_units:
                continue
            assert np.array_equal(res["fetch"][u], oo["fetch"][g]), (b, g, "fetch list")
            assert int(res["fetch_count"][u]) == oo["fetch"][g].size
            assert int(res["h2d_count"][u]) == oo["h2d"][g].size
        for h in range(hq):
            row = b * hq + h
            if (b, h // G) in exempt_units:
                continue
            e = rel_l2(res["o"][row], oo["o"][h])
            worst = max(worst, e)
            assert e <= tol, (b, h, "o", e)
            assert rel_l2(res["n_hat"][row], oo["n_hat"][h]) <= tol, (b, h, "n_hat")
            assert abs(res["d_hat"][row] - oo["d_hat"][h]) <= tol * oo["d_hat"][h], (b, h, "d_hat")
            assert abs(res["lse"][row] - oo["lse"][h]) <= tol, (b, h, "lse")
            np.testing.assert_allclose(res["eps_after"][row], oo["eps_after"][h], rtol=1e-9,
                                       atol=1e-15)
    return dict(worst_o=worst, exempt=len(exempt_units),
                fetched=int(np.sum(res["fetch_count"])), h2d=int(np.sum(res["h2d_count"])),
                certified=int(np.sum(res["certified"])))


def session(wl, **kw):
    from long_context_decode_kvfetch_amd.runner import Session
    return Session(wl, **kw)


def run_parity(wl, steps=(0,), label="", kappa=None, eps=None, delta=None, sketch_of=None,
               resolved=None, **kw):
    """Compress `wl` on the GPU, compare the state with the oracle's, run `steps` decode
    steps (each followed by verkv_check) and compare every one; returns (session, summaries)."""
    from long_context_decode_kvfetch_amd import verkv
    say(f"[parity] {label}: {wl.name}")
    sess = session(wl, **kw)
    sess.compress()
    ocomp = oracle_compress(wl)
    compare_state(sess, wl, ocomp)
    summ = []
    for st in steps:
        q = sess.queries(st)
        say(f"[parity] {label}: step {st}")
        sess.step(q, kappa=kappa, eps=eps, delta=delta, resolved=resolved is not None)
        verkv.check(sess.shape, sess.cap, sess.dws)
        oo = oracle_step(wl, ocomp, st, kappa=kappa, eps=eps, delta=delta, sketch_of=sketch_of,
                         resolved=resolved)
        summ.append(compare_step(sess, wl, ocomp, oo, st, kappa=kappa, eps=eps, delta=delta,
                                 sketch_of=sketch_of, resolved=resolved))
    say(f"[parity] {label}: {summ}")
    return sess, summ
