"""GPU parity of the re-solved reading of eqs. (9)-(10) (verkv_decode_step_ex with
VERKV_STEP_RESOLVED: the fetch order of eq. (9) with lambda frozen, the k* cut with the
bias of Definition 2 solved on each candidate set) against the oracle's
decide_head_resolved.  On small rows the oracle finds k* by the literal scan of eq. (10)
over k; on large ones by bisection over k, which test_oracle_resolved.py pins to the scan
(eps_hat of the re-solved reading is non-increasing in k).  Fetch lists, k*, the kept
set's bias and every output are compared to the usual standard."""
import numpy as np
import pytest

from long_context_decode_kvfetch_amd import synth
from parity_util import require_gpu_library, run_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu_library()


def test_resolved_small_rows_against_the_scan():
    """n = 2500 (one decision workgroup per row) and n = 4096 with two workgroups per row,
    bf16 and float32 caches, the oracle's k* by the scan over k."""
    _, s1 = run_parity(synth.gqa_layer(seed=80, n=2500, steps=1, hkv=1, n_local=64),
                       label="resolved n=2500", resolved="scan")
    _, s2 = run_parity(synth.single_head(81, n=4096), label="resolved single head", resolved="scan")
    assert s1[0]["fetched"] > 0 and s2[0]["fetched"] > 0


def test_resolved_fetches_less_than_frozen_on_the_gqa_recipe():
    """n = 8192, 2 KV heads x 4 rows: the re-solved cut against the oracle (bisection), and
    its union F against the frozen reading's on the same step."""
    wl = synth.gqa_layer(seed=82, n=8192, steps=1, hkv=2)
    _, sr = run_parity(wl, label="resolved gqa 8K", resolved="bisect")
    _, sf = run_parity(wl, label="frozen gqa 8K")
    say(f"[resolved] union F: re-solved {sr[0]['fetched']}, frozen {sf[0]['fetched']}")
    assert sr[0]["fetched"] < sf[0]["fetched"]


def test_resolved_full_size_layer():
    """The 32K GQA layer (32 rows, a team of workgroups per row with the slice in
    registers and LDS)."""
    run_parity(synth.gqa_layer(0, steps=1), label="resolved 32K", resolved="bisect")


def test_resolved_streamed_slices():
    """Slices too long for the register and LDS caches: one 40K-token sequence (a team
    per row) and 16 sequences of 5K-6K tokens (one workgroup per row, 512 rows)."""
    run_parity(synth.gqa_layer(seed=83, n=40000, steps=1), label="resolved 40K", resolved="bisect")
    wl = synth.ragged_batch(seed=84, batch=16, n_min=5000, n_max=6000, steps=1)
    run_parity(wl, label="resolved 16 x 5K", resolved="bisect")


def test_resolved_other_kappa_and_tolerances():
    wl = synth.gqa_layer(seed=85, n=4096, steps=1, hkv=2)
    run_parity(wl, label="resolved kappa 4", kappa=4.0, resolved="bisect")
    run_parity(wl, label="resolved eps 0.2 delta 0.3", eps=0.2, delta=0.3, resolved="bisect")
    # kappa = 0 and infinity: lambda does not depend on the bias, the readings coincide
    run_parity(wl, label="resolved kappa inf", kappa=float("inf"), resolved="bisect")
    run_parity(wl, label="resolved kappa 0", kappa=0.0, resolved="bisect")


def test_resolved_exact_ties():
    """Tied fetch keys across the cut (two groups of identical keys with equal scores):
    the search runs into the token-index digits."""
    from test_gpu_edges import _tied
    wl = _tied(synth.gqa_layer(seed=86, n=8192, steps=1, hkv=2), 2, 5)
    _, summ = run_parity(wl, label="resolved ties", resolved="bisect")
    assert summ[0]["fetched"] > 0
