"""GPU parity of the growing cache (verkv_append) against the oracle's append step
(oracle/api.py: append_sequence): after every few appended tokens the inclusion
probabilities (float64 bits), the resident mask and the pivot lists must be identical,
and a decode step on the grown cache must meet the usual parity standard (which also
checks the pivot K/V rows the append re-laid out: the resident-pivot attention reads
them).  The pages compress the cache once, at prefill; the append reading is the
library's, so these tests pin the GPU to the oracle's reading, not to the pages."""
import numpy as np
import pytest
import torch

from long_context_decode_kvfetch_amd import synth
from oracle import api as oapi
from parity_util import (compare_state, compare_step, oracle_compress, oracle_step,
                         require_gpu_library, say, session)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu_library()


def _new_tokens(wl, rng):
    """Rows and scores of one appended token per (sequence, KV head): keys and values
    ~ N(0, 1) held exactly by the cache dtype, scores ~ Beta(0.3, 3)."""
    B, hkv = wl.batch, wl.n_kv_heads
    k = rng.standard_normal((B, hkv, 128), dtype=np.float32)
    v = rng.standard_normal((B, hkv, 128), dtype=np.float32)
    if wl.kv_dtype == "bf16":
        k, v = synth.round_bf16(k), synth.round_bf16(v)
    tau = rng.beta(0.3, 3.0, size=(B, hkv)).astype(np.float32)
    return k, v, tau


def _grow_oracle(wl, ocomp, k, v, tau):
    for b, s in enumerate(wl.seqs):
        ocomp[b] = oapi.append_sequence(ocomp[b], tau[b], wl.n_sink, wl.n_local, wl.layer, b,
                                        wl.seed)
        s.K = np.concatenate([s.K, k[b][:, None]], axis=1)
        s.V = np.concatenate([s.V, v[b][:, None]], axis=1)
        s.tau = np.concatenate([s.tau, tau[b][:, None]], axis=1)
        s.n += 1


def _grow_and_check(wl, appends, label, check_every=8, seed=0, step_before=True):
    rng = np.random.default_rng([seed, 1234])
    sess = session(wl, grow=appends)
    sess.compress()
    ocomp = oracle_compress(wl)
    compare_state(sess, wl, ocomp)
    if step_before:                                  # stages host rows of the old shape
        sess.step(sess.queries(0))
    for i in range(appends):
        k, v, tau = _new_tokens(wl, rng)
        st = sess.append(k, v, tau)
        _grow_oracle(wl, ocomp, k, v, tau)
        if (i + 1) % check_every == 0 or i + 1 == appends:
            torch.cuda.synchronize()
            assert int(st.item()) == 0, (label, i, int(st.item()))
            compare_state(sess, wl, ocomp)
            say(f"[append] {label}: {i + 1} tokens appended, state identical")
    from long_context_decode_kvfetch_amd import verkv
    sess.step(sess.queries(0))
    verkv.check(sess.shape, sess.cap, sess.dws)
    oo = oracle_step(wl, ocomp, 0)
    summ = compare_step(sess, wl, ocomp, oo, 0)
    say(f"[append] {label}: decode step after the appends {summ}")
    return sess, ocomp, summ


def test_append_window_departures_include_appended_tokens():
    """A 16-token local window and 40 appends: from the 17th append on, the token leaving
    the window is one appended earlier."""
    wl = synth.gqa_layer(seed=70, n=4096, steps=1, hkv=2, n_local=16, eta=1.0 / 8)
    _, ocomp, summ = _grow_and_check(wl, 40, "window 16")
    assert summ["fetched"] > 0
    assert all(c.rule == "water" for c in ocomp[0])


def test_append_ragged_batch():
    """Three sequences of different lengths grow together; every head's pivot rows move
    to the new schedule."""
    wl = synth.ragged_batch(seed=71, batch=3, n_min=1500, n_max=5000, n_local=8)
    _grow_and_check(wl, 24, "ragged", seed=1)


def test_append_without_local_window():
    """n_local = 0: the appended token itself takes the rule and its own draw."""
    wl = synth.gqa_layer(seed=72, n=3000, steps=1, hkv=2, n_local=0)
    _grow_and_check(wl, 20, "no window", seed=2)


def test_append_no_budget_branch_drops_departing_tokens():
    """The prefill's budget was exactly the forced tokens (r = 0 elsewhere): every token
    leaving the window gets r = 0 and leaves the pivot list."""
    wl = synth.gqa_layer(seed=73, n=4096, steps=1, hkv=2, n_local=60, eta=1.0 / 64)
    sess, ocomp, _ = _grow_and_check(wl, 12, "no budget", seed=3)
    assert all(c.rule == "none" for c in ocomp[0])
    for h in sess.state_numpy():
        assert h["piv_count"] == 64


def test_append_saturated_branch():
    wl = synth.gqa_layer(seed=74, n=4096, steps=1, hkv=2, eta=0.25)
    tau = wl.seqs[0].tau
    rng = np.random.default_rng(6)
    for g in range(2):
        keep = rng.choice(np.arange(4, 4096 - 128), size=100, replace=False)
        t = np.zeros(4096, np.float32)
        t[keep] = tau[g, keep]
        tau[g] = t
    _, ocomp, _ = _grow_and_check(wl, 10, "saturated", seed=4)
    assert all(c.rule == "saturated" for c in ocomp[0])


def test_append_beyond_pivot_capacity_changes_nothing():
    """eta = 1 (every token resident): with the pivot capacity exactly the prefill's
    count, the first append would overflow it; the status word says so (8) and the state
    is left as it was."""
    wl = synth.gqa_layer(seed=75, n=2000, steps=1, hkv=2, eta=1.0, n_local=16)
    sess = session(wl, grow=4, cap=2000)
    sess.compress()
    before = sess.state_numpy()
    old_shape = sess.shape
    k, v, tau = _new_tokens(wl, np.random.default_rng(9))
    st = sess.append(k, v, tau)
    torch.cuda.synchronize()
    assert int(st.item()) == 8
    sess.shape = old_shape
    after = sess.state_numpy()
    for x, y in zip(before, after):
        assert np.array_equal(x["r"].view(np.uint64), y["r"].view(np.uint64))
        assert np.array_equal(x["resident"], y["resident"])
        assert np.array_equal(x["piv_idx"], y["piv_idx"]) and x["piv_count"] == y["piv_count"]
