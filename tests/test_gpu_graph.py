"""A decode step captured into a HIP graph (torch.cuda.CUDAGraph drives the capture on
its own stream) and replayed: verkv_decode_step + verkv_refine on a caller workspace,
whose refine forks onto the library's second stream and joins it back, and
verkv_step_noalloc, whose kernels all run on the caller's stream.  No call of a step
enqueues a memset or a host synchronisation, so the graph holds kernel nodes and the
fork/join only.  Every replay must give the eagerly launched step's outputs bit for bit;
replays are separated by eager steps on other queries and synchronisations, and new
queries are copied into the captured query buffer before each replay."""
import numpy as np
import pytest
import torch

from long_context_decode_kvfetch_amd import synth
from parity_util import require_gpu_library, say, session

pytestmark = pytest.mark.gpu

KEYS = ("m_hat", "d_sketch", "beta_star", "eps_hat", "certified", "kstar", "eps_after",
        "d_hat", "lse", "fetch_count", "h2d_count", "o", "n_hat")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu_library()


def _same(got, ref, label):
    for k in KEYS:
        assert np.array_equal(got[k], ref[k]), (label, k)
    for a, b in zip(got["fetch"], ref["fetch"]):
        assert np.array_equal(a, b), label


def _replays(sess, run_eager, capture, label):
    from long_context_decode_kvfetch_amd import verkv
    qs = [sess.queries(i) for i in range(4)]
    refs = []
    for q in qs[:3]:
        refs.append(run_eager(q))
    qbuf = qs[0].clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture(qbuf)
    say(f"[graph] {label}: captured")
    for i in (0, 1, 2, 1):
        qbuf.copy_(qs[i])
        g.replay()
        torch.cuda.synchronize()
        got = sess.results_numpy(sess.gout)
        _same(got, refs[i], f"{label} replay of query {i}")
        run_eager(qs[3])                      # eager work between the replays
        torch.cuda.synchronize()
    verkv.check(sess.shape, sess.cap, sess.dws)
    say(f"[graph] {label}: 4 replays identical to the eager steps")


def test_graph_of_decode_step_and_refine():
    from long_context_decode_kvfetch_amd import verkv
    wl = synth.gqa_layer(seed=80, n=8192, steps=4, hkv=2)
    sess = session(wl)
    sess.compress()
    sess.gout = verkv.StepBuffers(sess.shape, fetch_cap=max(sess.shape.caps))

    def eager(q):
        sess.step(q)
        return sess.results_numpy()

    _replays(sess, eager, lambda qb: sess.step(qb, out=sess.gout), "decode + refine")


def test_graph_of_step_noalloc():
    from long_context_decode_kvfetch_amd import verkv
    wl = synth.gqa_layer(seed=81, n=6000, steps=4, hkv=2)
    sess = session(wl)
    sess.compress()
    sess.gout = verkv.StepBuffers(sess.shape, fetch_cap=max(sess.shape.caps))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    eout = verkv.StepBuffers(sess.shape, fetch_cap=max(sess.shape.caps))

    def noalloc(q, out):
        verkv.step_noalloc(sess.shape, sess.state, q, wl.kappa, wl.eps, wl.delta, sess.K_host,
                           sess.V_host, out, status)

    def eager(q):
        noalloc(q, eout)
        return sess.results_numpy(eout)

    _replays(sess, eager, lambda qb: noalloc(qb, sess.gout), "step_noalloc")
    assert int(status.item()) == 0
