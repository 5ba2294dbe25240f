"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from long_context_decode_kvfetch_amd import synth
from parity_util import (compare_state, compare_step, oracle_compress, oracle_step,
                         require_gpu_library, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu_library()


def _session(wl, **kw):
    from long_context_decode_kvfetch_amd.runner import Session
    return Session(wl, **kw)


def _run(wl, steps=(0,), label="", kappa=None, eps=None, delta=None, sketch_of=None, **kw):
    say(f"[parity] {label}: {wl.name}")
    sess = _session(wl, **kw)
    sess.compress()
    ocomp = oracle_compress(wl)
    compare_state(sess, wl, ocomp)
    summ = []
    for st in steps:
        q = sess.queries(st)
        say(f"[parity] {label}: step {st}")
        sess.step(q, kappa=kappa, eps=eps, delta=delta)
        from long_context_decode_kvfetch_amd import verkv
        verkv.check(sess.shape, sess.cap, sess.dws)
        oo = oracle_step(wl, ocomp, st, kappa=kappa, eps=eps, delta=delta, sketch_of=sketch_of)
        summ.append(compare_step(sess, wl, ocomp, oo, st, kappa=kappa, eps=eps, delta=delta,
                                 sketch_of=sketch_of))
    say(f"[parity] {label}: {summ}")
    return sess, summ


def test_single_head_fp32_g8():
    """n=4096, 1 KV head, 8 query rows, fp32 cache, eta=1/8."""
    _run(synth.single_head(0), label="single-head")


def test_single_head_other_seeds():
    for seed in (1, 2):
        _run(synth.single_head(seed), label=f"single-head seed {seed}")


def test_gqa_layer_full_size_bf16():
    """32 Q / 8 KV heads, n=32768, bf16, eta=1/16: two decode steps at full size."""
    _run(synth.gqa_layer(0, steps=2), steps=(0, 1), label="gqa-32k")


def test_ragged_tails_and_small_sequences():
    """Lengths that are not multiples of the sketch chunk or of 32-bit words, and
    several sequences (independent Philox stream ids)."""
    wl = synth.ragged_batch(seed=5, batch=3, n_min=1000, n_max=5000)
    wl.seqs[0] = synth.gqa_layer(seed=9, n=2333, steps=1).seqs[0]
    _run(wl, label="ragged")


def test_many_small_heads_pivot_runs_span_heads():
    """128 short sequences x 10 KV heads = 1280 heads of one or two 32-row pivot chunks
    each: the resident-pivot workers (768) each take chunks of two or three heads, so the
    kernel follows a head change inside a worker, including the third head it finds
    itself, and the finishing kernel sums several partial slots per head."""
    wl = synth.ragged_batch(seed=11, batch=128, n_min=400, n_max=700, n_local=16, hkv=10)
    _run(wl, label="many small heads")


def test_ragged_16_sequences_full_size_pivots_only():
    """The workload the pivotal-KV stream is timed on: 16 sequences with lengths uniform
    in [8K, 64K] (32q/8kv, bf16, eta = 1/16), eps large enough that every row certifies,
    so the estimator is the resident pivots alone, through the same persistent-worker
    launch (768 workers, runs spanning KV heads and sequences)."""
    wl = synth.ragged_batch(seed=0, batch=16, steps=3)
    _run(wl, steps=(2,), eps=1e9, label="ragged-16 pivots only")


def test_uniform_tau_no_heavy_hitters_certifies():
    """Uniform scores and no planted keys: eps_hat(L) is about 0.14 at eta = 1/16, so at
    eps = 0.2 every row certifies and nothing is fetched (the no-fetch path)."""
    wl = synth.gqa_layer(seed=1, n=32768, steps=1, hkv=2, tau_kind="uniform", hh_frac=0.0,
                         eps=0.2)
    _, summ = _run(wl, label="uniform")
    assert summ[0]["certified"] == wl.n_q_heads and summ[0]["fetched"] == 0


def test_eta_one_is_exact_attention():
    wl = synth.gqa_layer(seed=4, n=3000, steps=1, hkv=2, eta=1.0, n_local=16)
    sess, summ = _run(wl, label="eta=1")
    res = sess.results_numpy()
    assert np.all(res["certified"] == 1) and np.all(res["eps_hat"] == 0.0)
    s = wl.seqs[0]
    for h in range(wl.n_q_heads):
        q = torch.tensor(wl.queries[0, 0, h], dtype=torch.float64)
        K = torch.tensor(s.K[h // wl.group], dtype=torch.float64)
        V = torch.tensor(s.V[h // wl.group], dtype=torch.float64)
        ref = torch.softmax(K @ q / math.sqrt(128), 0) @ V
        err = float(torch.linalg.norm(torch.tensor(res["o"][h], dtype=torch.float64) - ref) /
                    torch.linalg.norm(ref))
        assert err < 2e-3


def test_tolerance_extremes_and_kappa_limits():
    wl = synth.single_head(3, n=2048)
    _run(wl, label="eps tiny", eps=1e-12)
    _run(wl, label="eps huge", eps=1e6)
    _run(wl, label="kappa inf", kappa=math.inf)
    _run(wl, label="kappa 0", kappa=0.0)
    _run(wl, label="kappa 4 delta 0.3", kappa=4.0, delta=0.3)


def test_deterministic_repeat():
    wl = synth.gqa_layer(seed=2, n=16384, steps=1, hkv=4)
    sess = _session(wl)
    sess.compress()
    q = sess.queries(0)
    say("[parity] determinism: first run")
    sess.step(q)
    a = sess.results_numpy()
    say("[parity] determinism: second run")
    sess.step(q)
    b = sess.results_numpy()
    for k in a:
        if k == "fetch":
            for x, y in zip(a[k], b[k]):
                assert np.array_equal(x, y)
        else:
            assert np.array_equal(a[k], b[k]), k


def test_host_fetch_reads_keys_when_sketch_not_exact():
    """With sketch_exact = 0 the refinement scores the fetched rows from the host keys."""
    _run(synth.single_head(5, n=4096), label="single-head, K from host", sketch_exact=False)
    _run(synth.gqa_layer(seed=6, n=8192, steps=1, hkv=2), label="gqa, K from host",
         sketch_exact=False)


def test_long_context_131k_eta_1_32():
    """n = 131072, eta = 1/32 (the long-context shape), two KV heads, full length."""
    _run(synth.gqa_layer(seed=7, n=131072, steps=1, hkv=2, eta=1.0 / 32, eps=0.1),
         label="131k")


def test_long_context_keys_planted_on_non_resident_tokens():
    """The long-context stress workload at full shape (n = 131072, 8 KV heads, eta = 1/32):
    2048 keys per KV head get the heavy-hitter direction on tokens the sampler did not keep
    (the resident mask comes from the oracle's PoissonComp, which the GPU reproduces bit for
    bit), so most of the attention mass sits on host-only tokens; eps = 0.3."""
    wl = synth.long_context(seed=0, n=131072, steps=1, eps=0.3)
    resident = np.stack([c.resident for c in oracle_compress(wl)[0]])
    synth.plant_adversarial(wl, resident, 2048)
    _run(wl, label="131k planted")


def test_tau_exactly_zero_on_part_of_the_cache():
    """Scores that are exactly 0 on about 30% of the tokens: those get r = 0, are never
    drawn and stay in L with lambda = 0 (pure bias, fetch candidates)."""
    wl = synth.gqa_layer(seed=21, n=8192, steps=1, hkv=2)
    tau = wl.seqs[0].tau
    tau[np.random.default_rng(99).random(tau.shape) < 0.3] = 0.0
    _run(wl, label="tau zeros")


def test_maximum_sequence_length():
    """n = 2^20 tokens, the longest sequence the library accepts (token ids fill the 20
    bits of a host-row list entry), one KV head of four query rows."""
    _run(synth.gqa_layer(seed=5, n=1 << 20, steps=1, hkv=1, eta=1.0 / 32, eps=0.1), label="n=2^20")


def test_philox_layer_word():
    """A later layer of a multi-layer decode (layer word 35 of the Philox counter)."""
    _run(synth.gqa_layer(seed=3, n=8192, steps=1, layer=35), label="layer 35")


@pytest.mark.parametrize("sketch_2bit,stage_slots", [(False, 0), (True, 0), (False, 8192), (True, 6000)],
                         ids=["exact sketch", "2-bit sketch", "exact sketch, 8192 slots",
                              "2-bit sketch, 6000 slots"])
def test_prefetch_and_workspace_history_do_not_change_results(sketch_2bit, stage_slots):
    """Three steps on one layer with the cross-step staging of host rows on, off, and on
    with a workspace that starts out as random bytes: every output is bit-identical (the
    staged rows are the same host rows; a foreign workspace only costs time).  With the
    2-bit sketch each row's key is staged beside its value (the host fetch scores fetched
    rows from the host keys there), and the staging copies must run on every step.  With
    8192 staging slots per KV head the host-row lists (about 5K rows per head here) carry
    slot numbers above 4095 in the bits the 8192-token capacity leaves free."""
    from long_context_decode_kvfetch_amd import verkv
    wl = synth.gqa_layer(seed=2, n=8192, steps=3, hkv=2)
    keys = ("o", "lse", "n_hat", "d_hat", "beta_star", "eps_hat", "kstar", "certified",
            "fetch_count", "h2d_count", "eps_after")
    runs = []
    for label, kw, scramble in (("prefetch", {}, False), ("no prefetch", {"prefetch": False}, False),
                                ("random workspace", {}, True)):
        say(f"[parity] history: {label}, {'2-bit' if sketch_2bit else 'exact'} sketch")
        kw = dict(kw, sketch_2bit=sketch_2bit, stage_slots=stage_slots)
        sess = _session(wl, **kw)
        sess.compress()
        if scramble:
            g = torch.Generator(device="cuda").manual_seed(7)
            sess.dws.copy_(torch.randint(0, 256, sess.dws.shape, dtype=torch.uint8, device="cuda",
                                         generator=g).view(sess.dws.dtype))
            torch.cuda.synchronize()
            try:
                verkv.check(sess.shape, sess.cap, sess.dws)      # clears random kernel flags
            except Exception:
                pass
        steps = []
        verkv.profile_begin(64)
        for st in range(3):
            sess.step(sess.queries(st))
            verkv.check(sess.shape, sess.cap, sess.dws)
            r = sess.results_numpy()
            steps.append({k: np.array(r[k]) for k in keys})
            # rows served from the staging area: none without staging or before a plan exists
            staged = sess.staged_rows()
            if "prefetch" in kw or st == 0:
                assert staged == 0, (label, st, staged)
            else:
                assert 0 < staged <= int(r["h2d_count"].sum()), (label, st, staged)
        launches = verkv.profile_report()["prefetch"][1]
        verkv.profile_end()
        assert launches == (0 if "prefetch" in kw else 3), (label, launches)
        runs.append(steps)
    for label, other in (("no prefetch", runs[1]), ("random workspace", runs[2])):
        for st in range(3):
            for k in keys:
                assert np.array_equal(runs[0][st][k], other[st][k]), (label, st, k)


def test_staged_rows_of_another_cache_are_not_reused():
    """One workspace used for two layers in turn (two host caches of the same shape):
    the staging header names the cache its rows came from, so a step of layer B on a
    workspace that layer A filled reads no row of A's cache; every output equals that of
    layer B on a workspace of its own, bit for bit."""
    from long_context_decode_kvfetch_amd import verkv
    keys = ("o", "lse", "n_hat", "d_hat", "eps_after", "fetch_count", "h2d_count")
    wa = synth.gqa_layer(seed=3, n=8192, steps=3, hkv=2, layer=0)
    wb = synth.gqa_layer(seed=3, n=8192, steps=3, hkv=2, layer=1)
    sa, sb, ref = _session(wa), _session(wb), _session(wb)
    for s_ in (sa, sb, ref):
        s_.compress()
    assert sa.dws.numel() == sb.dws.numel()
    sb.dws = sa.dws                                   # B borrows A's workspace
    expect = []
    for st in range(3):
        ref.step(ref.queries(st))
        r = ref.results_numpy()
        expect.append({k: np.array(r[k]) for k in keys})
    for st in range(3):
        say(f"[parity] shared workspace: step {st}")
        sa.step(sa.queries(st))                       # A stages rows of its own cache
        sb.step(sb.queries(st))                       # then B runs on the same workspace
        verkv.check(sb.shape, sb.cap, sb.dws)
        got = sb.results_numpy()
        for k in keys:
            assert np.array_equal(np.array(got[k]), expect[st][k]), (st, k)


def test_staging_slots_survive_evictions_and_cache_switches():
    """Eight steps on one workspace shared by two layers (two host caches of the same
    shape) in the order A A B A B B A A, with a staging area of 1500 rows per KV head
    against host-row lists of about 5K rows: every plan evicts and refills slots, and a
    plan made for one cache must not be carried out for the other.  Every output equals
    that of the same layer without staging, bit for bit; the staged copies run on every
    step (they do nothing when the pending plan names the other cache)."""
    from long_context_decode_kvfetch_amd import verkv
    keys = ("o", "lse", "n_hat", "d_hat", "eps_after", "fetch_count", "h2d_count", "kstar")
    wa = synth.gqa_layer(seed=4, n=8192, steps=8, hkv=2, layer=0)
    wb = synth.gqa_layer(seed=4, n=8192, steps=8, hkv=2, layer=1)
    sa, sb = _session(wa, stage_slots=1500), _session(wb, stage_slots=1500)
    ra, rb = _session(wa, prefetch=False), _session(wb, prefetch=False)
    for s_ in (sa, sb, ra, rb):
        s_.compress()
    sb.dws = sa.dws                                   # one staging area for both caches
    order = "AABABBAA"
    taken = {"A": 0, "B": 0}
    verkv.profile_begin(512)                          # room for every launch of the 16 steps
    for i, name in enumerate(order):
        sess, ref = (sa, ra) if name == "A" else (sb, rb)
        st = taken[name]
        taken[name] += 1
        say(f"[parity] staging slots: step {i} on cache {name} (its step {st})")
        sess.step(sess.queries(st))
        verkv.check(sess.shape, sess.cap, sess.dws)
        got = sess.results_numpy()
        got = {k: np.array(got[k]) for k in keys}
        ref.step(ref.queries(st))
        want = ref.results_numpy()
        for k in keys:
            assert np.array_equal(got[k], np.array(want[k])), (i, name, k)
        assert int(got["h2d_count"].sum()) > 2 * 1500          # the lists outgrow the area
    launches = verkv.profile_report()
    verkv.profile_end()
    assert launches["prefetch"][1] == len(order) and launches["stage_plan"][1] == len(order)


# ------------------------------------------------------------------ the 2-bit sketch
def _sketch2_of(K):
    """The oracle's 2-bit sketch of key rows exactly as the device holds them."""
    from oracle import sketch2
    return sketch2.sketch_of(K)


def _unpack_sketch2(raw):
    """Codes [rows][128], mn, sc [rows][4] from 64-byte rows (layout in include/verkv.h:
    word w = codes of dimensions 8w.. | codes of 8(w+8).. << 16; then (mn, sc) of groups
    0, 2, 1, 3 as float32)."""
    words = np.ascontiguousarray(raw[:, :32]).view("<u4")
    prm = np.ascontiguousarray(raw[:, 32:]).view("<f4")
    rows = raw.shape[0]
    codes = np.zeros((rows, 128), dtype=np.uint8)
    for piece in range(16):
        w = words[:, piece % 8] >> np.uint32(16 * (piece // 8))
        for e in range(8):
            codes[:, piece * 8 + e] = (w >> np.uint32(2 * e)) & np.uint32(3)
    pos = {0: 0, 2: 1, 1: 2, 3: 3}
    mn = np.stack([prm[:, 2 * pos[g]] for g in range(4)], axis=1)
    sc = np.stack([prm[:, 2 * pos[g] + 1] for g in range(4)], axis=1)
    return codes, mn, sc


def test_2bit_sketch_codes_match_the_oracle():
    """verkv_quantize_sketch against the oracle's quantiser, bf16 and float32 keys:
    every code and every float32 group parameter bit for bit."""
    from oracle import sketch2
    for wl in (synth.gqa_layer(seed=3, n=5000, steps=1, hkv=2),
               synth.single_head(6, n=3000)):
        say(f"[parity] 2-bit sketch codes: {wl.name}")
        sess = _session(wl, sketch_2bit=True)
        torch.cuda.synchronize()
        raw = sess.sketch.cpu().numpy().reshape(-1, 64)
        codes, mn, sc = _unpack_sketch2(raw)
        r = 0
        for s in wl.seqs:
            for g in range(wl.n_kv_heads):
                oc, om, osc = sketch2.quantize_rows(s.K[g])
                n = s.n
                assert np.array_equal(codes[r:r + n], oc), (g, "codes")
                assert np.array_equal(mn[r:r + n].view(np.uint32), om.view(np.uint32)), (g, "mn")
                assert np.array_equal(sc[r:r + n].view(np.uint32), osc.view(np.uint32)), (g, "sc")
                r += n
        assert r == raw.shape[0]


def test_decode_with_2bit_sketch():
    """Steps 1-5 with the 2-bit sketch (weights from x_hat, fetched rows scored from the
    host keys) against the oracle run on the same sketch keys: 8 query rows per KV head
    on float32 keys (16 lanes per row) and the GQA shape on bf16 keys (8 lanes)."""
    _run(synth.single_head(2, n=4096), label="single-head, 2-bit sketch", sketch_2bit=True,
         sketch_of=_sketch2_of)
    _run(synth.gqa_layer(seed=8, n=8192, steps=2, hkv=2), steps=(0, 1), label="gqa, 2-bit sketch",
         sketch_2bit=True, sketch_of=_sketch2_of)
