"""Whole-call mirrors of the library's entry points on numpy arrays.
Test infrastructure for the oracle only.

compress_sequence  PoissonComp for every KV head of one sequence (prefill)
append_sequence    one decode-time token appended to every KV head (growing cache)
decode_sequence    KVFetch steps 1-5 for every query row of one sequence

A sequence's KV head g uses Philox counter (token, g, layer, stream) with the
sequence's stream id; query row h belongs to KV head h // G.
"""
from __future__ import annotations

import numpy as np

from . import kvfetch, poissoncomp


def compress_sequence(tau, n_sink, n_local, eta, layer, stream, seed):
    """tau: [Hkv][n] float32 -> list of poissoncomp.Compressed, one per KV head."""
    return [poissoncomp.compress_head(tau[g], n_sink, n_local, eta, g, layer, stream, seed)
            for g in range(tau.shape[0])]


def append_sequence(comp, tau_new, n_sink, n_local, layer, stream, seed):
    """One decode-time token appended to every KV head of one sequence: comp is the list
    of poissoncomp.Compressed, tau_new [Hkv] the new token's scores."""
    return [poissoncomp.append_token(comp[g], float(tau_new[g]), n_sink, n_local, g, layer,
                                     stream, seed) for g in range(len(comp))]


def decode_sequence(K, V, comp, q_rows, group, kappa, eps, delta, K_sketch=None, resolved=None):
    """K, V: [Hkv][n][d]; q_rows: [Hkv*G][d].  Returns a dict of per-row arrays
    (m_hat, D, beta_star, eps_hat, certified, kstar, eps_after, n_hat, d_hat, o,
    lse) and per-KV-head lists fetch / h2d (ascending token ids).  resolved: None for the
    frozen reading of eq. (9)-(10), "scan" or "bisect" for the re-solved one."""
    hkv = K.shape[0]
    rows = []
    for g in range(hkv):
        qs = q_rows[g * group:(g + 1) * group]
        Ks = None if K_sketch is None else K_sketch[g]
        rows.append(kvfetch.decode_kv_head(qs, K[g], V[g], comp[g].r, comp[g].resident,
                                           kappa, eps, delta, Ks, resolved))
    keys = [k for k in rows[0] if k not in ("fetch", "h2d")]
    out = {k: np.concatenate([np.atleast_1d(r[k]) if np.ndim(r[k]) < 2 else r[k] for r in rows])
           for k in keys}
    out["n_hat"] = np.concatenate([r["n_hat"] for r in rows], axis=0)
    out["o"] = np.concatenate([r["o"] for r in rows], axis=0)
    out["fetch"] = [r["fetch"] for r in rows]
    out["h2d"] = [r["h2d"] for r in rows]
    return out
