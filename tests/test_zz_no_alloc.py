"""verkv_step_noalloc (the decode step and refinement on the library's static scratch,
for callers that cannot allocate) against verkv_decode_step + verkv_refine on a caller
workspace: the same kernels on the same inputs, so every output must agree bit for bit.
Two calls in a row, the second on a smaller shape, so the second finds the first one's
contents in the shared array; and a shape too large for the array is refused before any
work."""
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


def _compare(sess, wl):
    from long_context_decode_kvfetch_amd import verkv
    sess.compress()
    q = sess.queries(0)
    sess.step(q)
    verkv.check(sess.shape, sess.cap, sess.dws)
    ref = sess.results_numpy()
    out = verkv.StepBuffers(sess.shape)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    verkv.step_noalloc(sess.shape, sess.state, q, wl.kappa, wl.eps, wl.delta, sess.K_host,
                       sess.V_host, out, status)
    got = sess.results_numpy(out)
    assert int(status.item()) == 0
    for k in KEYS:
        assert np.array_equal(got[k], ref[k]), k
    for a, b in zip(got["fetch"], ref["fetch"]):
        assert np.array_equal(a, b)
    return got


def test_noalloc_matches_the_workspace_entry_points_twice():
    from long_context_decode_kvfetch_amd import verkv
    assert verkv.lib().verkv_noalloc_scratch_bytes() == 64 << 20
    big = synth.gqa_layer(seed=60, n=8192, steps=1, hkv=2)
    say("[no-alloc] first call: 8 query rows, n = 8192")
    got = _compare(session(big), big)
    assert int(np.sum(got["fetch_count"])) > 0
    small = synth.gqa_layer(seed=61, n=3000, steps=1, hkv=1, group=8, kv_dtype="f32")
    say("[no-alloc] second call: smaller shape, n = 3000")
    _compare(session(small), small)


def test_noalloc_refuses_shapes_beyond_the_array():
    from long_context_decode_kvfetch_amd import verkv
    wl = synth.gqa_layer(seed=62, n=4096, steps=1, hkv=2)
    sess = session(wl)
    sess.compress()
    # 2^20 tokens x 8 KV heads x 4 rows: 256 MiB of sketch weights alone
    huge = verkv.LayerShape([1 << 20], 8, 4, wl.n_sink, wl.n_local, "bf16")
    out = verkv.StepBuffers(sess.shape)
    out.kstar.fill_(-7)
    torch.cuda.synchronize()
    with pytest.raises(verkv.VerKVError) as ei:
        verkv.step_noalloc(huge, sess.state, sess.queries(0), 1.0, 0.05, 0.05, sess.K_host,
                           sess.V_host, out)
    assert ei.value.status == verkv.EWORKSPACE and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out.kstar == -7)
