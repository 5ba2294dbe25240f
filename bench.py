"""Benchmark: certified KVFetch decode steps/s at 32K context, eta = 1/16, on one MI355X.

Workload (synthetic, seeded): Qwen3-4B-shaped decode, one layer per step: 32 query /
8 KV heads, head_dim 128, n = 32768, bf16 cache ~ N(0,1) with 1% planted heavy hitters
per KV head, tau ~ Beta(0.3, 3), eta = 1/16, H = 4 sink + 128 local, eps = 0.05,
delta = 0.05, one query token per step.  The complete K/V cache of every layer sits in
pinned host memory; the sketch (exact: the keys) and H u S are GPU resident.

A step is one verkv_decode_step + verkv_refine on one layer: sketch scores, shrinkage
fixed point, certificate, fetch selection, resident-pivot attention, host fetch of
F minus S over the host link, and the finished output; after it every query row is
certified (eps_hat(L minus F) < eps).  Steps run back to back on one stream, as decode
steps must.  Consecutive steps visit different layers (8 independently generated
layers, each with its own cache and queries) so that the working set of a step is not
served from the previous step's Infinity Cache lines.

Prints ONE JSON line.  --gpus N with N > 1 exits with a message: the benchmark measures
one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
N_CTX = 32768
ETA = 1.0 / 16
N_LAYERS_ROT = 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--layers", type=int, default=N_LAYERS_ROT)
    p.add_argument("--profile-steps", type=int, default=64)
    p.add_argument("--cpu-steps", type=int, default=8)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-pivot-batch", action="store_true",
                   help="skip the pivotal-stream measurement at the 16-sequence batch")
    p.add_argument("--no-resolved", action="store_true",
                   help="skip the leg with the re-solved reading of eqs. (9)-(10)")
    p.add_argument("--no-nofetch", action="store_true",
                   help="skip the no-fetch control leg (uniform scores, eps = 0.2)")
    p.add_argument("--no-gather", action="store_true",
                   help="skip the host-fetch comparison (zero-copy kernel against memcpy per run)")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the leg replaying each layer-step as a captured HIP graph")
    p.add_argument("--no-staging", action="store_true",
                   help="skip the sweep over the staging slots per KV head")
    p.add_argument("--no-2bit", action="store_true",
                   help="skip the 2-bit sketch leg (the same layers with a 2-bit key sketch)")
    p.add_argument("--sweep", action="store_true",
                   help="eta in {1/8, 1/16, 1/32} x eps in {0.01, 0.02, 0.05, 0.1, 0.3, 0.5} over the rotated "
                        "32K layers: steps/s and host traffic per setting, one JSON line")
    p.add_argument("--pivot-only", action="store_true",
                   help="time only the resident-pivot attention at the 16-sequence batch "
                        "and print its figures as one JSON line")
    p.add_argument("--no-decode36", action="store_true",
                   help="skip the 36-layer decode leg of the default run")
    p.add_argument("--no-long-context", action="store_true",
                   help="skip the 131072-token stress leg of the default run")
    p.add_argument("--decode36", action="store_true",
                   help="36 independent 32K layers decoded one after another per token "
                        "(eta=1/16, eps=0.05): tokens/s and host bytes per token, one JSON line")
    p.add_argument("--decode36-grid", action="store_true",
                   help="the 36-layer decode over eta in {1/8, 1/16, 1/32} x eps in {0.02, 0.05, 0.1} "
                        "(8 tokens each): tokens/s and host bytes per token, one JSON line")
    p.add_argument("--long-context", action="store_true",
                   help="one 131072-token sequence, eta=1/32, keys planted on non-resident "
                        "tokens, eps in {0.05, 0.1, 0.2, 0.3, 0.5}: steps/s and fetched share, one JSON line")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a 256 MiB elementwise copy kernel (HBM counter calibration)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def h2d_bandwidth(torch, nbytes=256 << 20, reps=5):
    """Pinned host -> device copy bandwidth, GB/s (contiguous)."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


# Counter-derived HBM traffic of the roofline kernel, written from two rocprofv3 --pmc
# runs (FETCH_SIZE, WRITE_SIZE) scaled by a copy kernel of known size.  The record
# carries a hash of the kernel's sources; once they change the figure no longer
# describes the kernel and traffic is reported as null.
KERNEL_SOURCES = {
    "sketch_scores": ("profiles/sketch_scores_gqa32k_traffic.md",
                      ("long_context_decode_kvfetch_amd/csrc/k_sketch.hip",
                       "long_context_decode_kvfetch_amd/csrc/kernels.h",
                       "long_context_decode_kvfetch_amd/csrc/common.h")),
    "attend_pivots": ("profiles/attend_pivots_ragged16_kernel_trace.md",
                      ("long_context_decode_kvfetch_amd/csrc/k_attend.hip",
                       "long_context_decode_kvfetch_amd/csrc/kernels.h",
                       "long_context_decode_kvfetch_amd/csrc/common.h")),
}

# Algorithmic bytes of the layer-step's HBM streams (the sketch is exact: the keys).
SKETCH_ROW_BYTES = 128 * 2          # bf16 key row per (KV head, token)
R_BYTES = 8                         # r_i, float64
PIVOT_ROW_BYTES = 2 * 128 * 2 + 8   # bf16 K and V rows of a pivot, plus its token index and r
WHAT_SCRATCH_BYTES = 4 * 8          # float64 sketch weights of G = 4 query rows (scratch)


def sketch_bytes(n_tok_heads):
    """The sketch stream: one key row and r per (KV head, token)."""
    return n_tok_heads * (SKETCH_ROW_BYTES + R_BYTES)


def step_algorithmic_bytes(n_tok_heads, pivot_rows):
    """Whole layer-step: the sketch stream, the pivotal stream, and the resident and fetch
    bitmasks (one bit per (KV head, token) each); query and output rows are negligible."""
    return sketch_bytes(n_tok_heads) + pivot_rows * PIVOT_ROW_BYTES + 2 * n_tok_heads // 8


def fail_on_flags(sessions, what):
    """verkv_check on every session's workspace: a step whose team barrier timed out or
    whose fixed point did not converge must not be counted, so the run stops here."""
    from long_context_decode_kvfetch_amd import verkv
    for sess in sessions:
        try:
            verkv.check(sess.shape, sess.cap, sess.dws)
        except verkv.VerKVError as e:
            print(f"bench.py: kernel flags after {what}: {e}", file=sys.stderr)
            sys.exit(3)


def timed(torch, run, first, count):
    """Run steps first .. first+count-1 back to back on the current stream with an event
    after each: (total ms, per-step ms list)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
    ev[0].record()
    for i in range(count):
        run(first + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(count)]
    return ev[0].elapsed_time(ev[count]), per


def percentiles(per):
    import numpy as np
    a = np.asarray(per, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel][1]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kernel):
    """Bytes per launch from the committed counter summary, or None if stale/absent."""
    try:
        with open(os.path.join(ROOT, KERNEL_SOURCES[kernel][0])) as f:
            lines = [l for l in f if l.startswith("traffic-record:")]
    except OSError:
        return None
    for line in lines:
        kv = dict(item.split("=", 1) for item in line.split()[1:])
        if kv.get("kernel") == kernel and kv.get("sources_sha256") == sources_sha256(kernel):
            return int(float(kv["traffic_bytes"]))
    return None


def pivotal_stream(torch, steps=8, fetch_steps=8):
    """The 16-sequence ragged batch (lengths uniform in [8K, 64K], 32q/8kv, bf16,
    eta = 1/16), two measurements on one compressed batch:
      * the resident-pivot attention (the pivotal-KV stream) timed on its own: eps large
        enough that every row certifies, so no host rows share the step; bytes,
        microseconds and GB/s per launch (dispatch-stamped events);
      * the batch at its stated tolerance eps = 0.05: steps/s with fetching (one decision
        workgroup per query row), fetched share and host bytes per step."""
    import numpy as np
    from long_context_decode_kvfetch_amd import synth, verkv
    from long_context_decode_kvfetch_amd.runner import Session
    wl = synth.ragged_batch(seed=0, batch=16, steps=steps + fetch_steps + 4)
    sess = Session(wl)
    sess.compress()
    qdev = torch.from_numpy(np.ascontiguousarray(wl.queries)).to("cuda")
    for i in range(2):
        sess.step(qdev[i], eps=1e9)
    torch.cuda.synchronize()
    verkv.profile_begin(16 * steps + 16)
    for i in range(2, steps + 2):
        sess.step(qdev[i], eps=1e9)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    fail_on_flags([sess], "the pivotal-stream leg")
    ms, cnt = prof["attend_pivots"]
    us = ms / cnt * 1e3
    rows = int(sess.state.piv_count.sum().item())
    nbytes = rows * 2 * 128 * 2
    # algorithmic bytes per pivot row: its bf16 K and V rows (512 B) plus its token index
    # and r (8 B); the kernel reads the estimator coefficients (4 B per query row) in
    # place of index and r
    alg = rows * PIVOT_ROW_BYTES
    piv = {"workload": "16 sequences, n ~ U[8K, 64K], 32q/8kv, d=128, bf16, eta=1/16, "
                       "every row certified (pivots only)",
           "pivot_rows": rows, "kv_bytes": nbytes, "algorithmic_bytes": alg,
           "avg_us": round(us, 2),
           "GBps": round(alg / (us * 1e-6) / 1e9, 1), "peak_GBps": HBM_PEAK_GBS,
           "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "kv_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
           "traffic": profiled_traffic("attend_pivots")}

    # the same batch at eps = 0.05
    base = steps + 2
    sess.step(qdev[base])                          # primes the cross-step staging
    torch.cuda.synchronize()
    ms, per = timed(torch, lambda i: sess.step(qdev[i]), base + 1, fetch_steps)
    fail_on_flags([sess], "the 16-sequence leg at eps = 0.05")
    sess.step(qdev[base + 1 + fetch_steps])
    r = sess.results_numpy()
    assert np.all(r["eps_after"] < wl.eps), "a row finished uncertified"
    ntok = sum(s.n for s in wl.seqs) * wl.n_kv_heads
    piv["eps_0_05"] = {"eps": wl.eps, "steps": fetch_steps,
                       "steps_per_s": round(fetch_steps / (ms * 1e-3), 2),
                       "ms_per_step": round(ms / fetch_steps, 3), "step_ms": percentiles(per),
                       "rows_certified_without_fetch": float(r["certified"].mean()),
                       "fetched_fraction_of_cache": int(r["fetch_count"].sum()) / ntok,
                       "h2d_fraction_of_cache": int(r["h2d_count"].sum()) / ntok,
                       "h2d_bytes_per_step": int(r["h2d_count"].sum()) * 128 * 2}
    del sess
    torch.cuda.empty_cache()
    return piv


def resolved_leg(torch, sessions, K=64, W=8, P=16):
    """The same rotated 32K layers with the re-solved reading of eqs. (9)-(10) (the bias
    solved on each candidate set of the k* cut, verkv_decode_step_ex): steps/s, what is
    fetched and what crosses the host link, and the kernel times."""
    import numpy as np
    from long_context_decode_kvfetch_amd import verkv
    L = len(sessions)
    per_layer = sessions[0].qdev.shape[0]

    def run(i):
        s2 = sessions[i % L]
        s2.step(s2.qdev[(i // L) % per_layer], resolved=True)

    for i in range(W):
        run(i)
    torch.cuda.synchronize()
    ms, per = timed(torch, run, W, K)
    fail_on_flags(sessions, "the re-solved reading leg")
    verkv.profile_begin(9 * P + 16)
    for i in range(W + K, W + K + P):
        run(i)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    cert = fetched = h2d = nrow = 0
    for s2 in sessions:
        s2.step(s2.qdev[0], resolved=True)
        r = s2.results_numpy()
        assert np.all(r["eps_after"] < s2.wl.eps), "a row finished uncertified"
        cert += int(r["certified"].sum())
        fetched += int(r["fetch_count"].sum())
        h2d += int(r["h2d_count"].sum())
        nrow += r["certified"].size
    ntok = L * N_CTX * 8
    return {"workload": "the rotated 32K GQA layers of the headline line, re-solved reading",
            "steps": K, "steps_per_s": round(K / (ms * 1e-3), 2), "ms_per_step": round(ms / K, 4),
            "step_ms": percentiles(per), "rows_certified_without_fetch": cert / nrow,
            "fetched_fraction_of_cache": fetched / ntok, "h2d_fraction_of_cache": h2d / ntok,
            "h2d_bytes_per_step": h2d / L * 128 * 2,
            "kernel_avg_us": {k: round(v[0] / v[1] * 1e3, 2) for k, v in prof.items() if v[1]}}


def no_fetch_leg(torch, L, K=64, W=8):
    """Control: the 32K GQA layer-step with uniform scores and no planted keys at
    eps = 0.2, where every row certifies without fetching (eps_hat(L) is about 0.14 at
    eta = 1/16): the step is the sketch stream, the decision and the resident pivots,
    with no host traffic.  Steps/s and the per-kernel times over rotated layers."""
    import numpy as np
    from long_context_decode_kvfetch_amd import synth, verkv
    from long_context_decode_kvfetch_amd.runner import Session
    per_layer = (K + W + 16 + L) // L + 1
    sess = []
    for layer in range(L):
        wl = synth.gqa_layer(seed=1, n=N_CTX, steps=per_layer, layer=layer, tau_kind="uniform",
                             hh_frac=0.0, eps=0.2)
        s2 = Session(wl)
        s2.compress()
        s2.qdev = torch.from_numpy(np.ascontiguousarray(wl.queries)).to("cuda")
        for sq in wl.seqs:
            sq.K = sq.V = None
        sess.append(s2)

    def run(i):
        s2 = sess[i % L]
        s2.step(s2.qdev[(i // L) % per_layer])

    for i in range(W):
        run(i)
    torch.cuda.synchronize()
    ms, per = timed(torch, run, W, K)
    fail_on_flags(sess, "the no-fetch leg")
    verkv.profile_begin(8 * 16 + 16)
    for i in range(W + K, W + K + 16):
        run(i)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    cert = nrow = fetched = 0
    for s2 in sess:
        s2.step(s2.qdev[0])
        r = s2.results_numpy()
        cert += int(r["certified"].sum())
        nrow += r["certified"].size
        fetched += int(r["fetch_count"].sum())
    kern = {k: round(v[0] / v[1] * 1e3, 2) for k, v in prof.items() if v[1]}
    piv_rows = sum(int(s2.state.piv_count.sum().item()) for s2 in sess) / L
    alg = step_algorithmic_bytes(8 * N_CTX, piv_rows)
    out = {"workload": "gqa decode layer-step: 32q/8kv, d=128, n=32768, bf16, exact sketch, "
                       "eta=1/16, tau uniform, no planted keys, eps=0.2, delta=0.05, layers rotated",
           "steps": K, "steps_per_s": round(K / (ms * 1e-3), 2), "ms_per_step": round(ms / K, 4),
           "step_ms": percentiles(per), "rows_certified_without_fetch": cert / nrow,
           "fetched_tokens": fetched, "step_algorithmic_bytes": int(alg),
           "step_GBps": round(alg / (ms / K * 1e-3) / 1e9, 1), "kernel_avg_us": kern}
    del sess
    torch.cuda.empty_cache()
    return out


def staging_leg(torch, wls, qdevs, K=64, W=8, slots=(2048, 4096, 16384, 32768)):
    """The 32K GQA layer-step over the rotated layers with the cross-step staging sized at
    `slots` rows per KV head (the library's default is 8192 here): steps/s, the device
    memory the staging area takes per layer (bf16 value rows), and the host-row kernel's
    time.  More slots keep more of the previous step's host rows on the device, at the
    cost of device memory the method otherwise keeps free."""
    from long_context_decode_kvfetch_amd import verkv
    from long_context_decode_kvfetch_amd.runner import Session
    out = {"workload": "the rotated 32K GQA layers of the headline line", "settings": []}
    for ns in slots:
        sess = []
        for wl, q in zip(wls, qdevs):
            s2 = Session(wl, stage_slots=ns)
            s2.compress()
            s2.qdev = q
            sess.append(s2)
        L = len(sess)
        per = qdevs[0].shape[0]

        def run(i):
            s2 = sess[i % L]
            s2.step(s2.qdev[(i // L) % per])
        W0 = max(W + L, 2 * L)                # at least two steps per layer: staging primed
        for i in range(W0):
            run(i)
        torch.cuda.synchronize()
        ms, per_step = timed(torch, run, W0, K)
        fail_on_flags(sess, f"the staging leg at {ns} slots")
        verkv.profile_begin(16 * 16 + 16)
        for i in range(W0 + K, W0 + K + 16):
            run(i)
        torch.cuda.synchronize()
        prof = verkv.profile_report()
        verkv.profile_end()
        out["settings"].append({
            "stage_slots": ns, "steps_per_s": round(K / (ms * 1e-3), 2),
            "step_ms": percentiles(per_step),
            "staging_bytes_per_layer": 8 * ns * 128 * 2,
            "host_rows_us": round(prof["attend_host"][0] / prof["attend_host"][1] * 1e3, 1),
            "prefetch_us": round(prof["prefetch"][0] / max(1, prof["prefetch"][1]) * 1e3, 1),
            "decide_us": round(prof["decide"][0] / prof["decide"][1] * 1e3, 1)})
        log(f"[bench] staging {ns} slots: {out['settings'][-1]['steps_per_s']} steps/s")
        del sess
        torch.cuda.empty_cache()
    return out


def graph_leg(torch, sessions, K=64, W=8):
    """The 32K layer-step (verkv_decode_step + verkv_refine, staging on) captured once per
    layer into a HIP graph and replayed over the rotated layers, against the same steps
    launched kernel by kernel; both copy the step's queries into the layer's query buffer
    first.  Steps/s and per-step percentiles of both."""
    from long_context_decode_kvfetch_amd import verkv
    L = len(sessions)
    per = sessions[0].qdev.shape[0]
    qbuf = [s.qdev[0].clone() for s in sessions]
    for s, qb in zip(sessions, qbuf):
        s.step(qb)
    torch.cuda.synchronize()
    graphs = []
    for s, qb in zip(sessions, qbuf):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.step(qb)
        graphs.append(g)

    def run_graph(i):
        j = i % L
        qbuf[j].copy_(sessions[j].qdev[(i // L) % per])
        graphs[j].replay()

    def run_eager(i):
        j = i % L
        qbuf[j].copy_(sessions[j].qdev[(i // L) % per])
        sessions[j].step(qbuf[j])

    out = {"workload": "the rotated 32K GQA layers of the headline line, one graph per layer"}
    for name, run in (("eager", run_eager), ("graph", run_graph), ("eager_again", run_eager)):
        for i in range(W):
            run(i)
        torch.cuda.synchronize()
        ms, per_step = timed(torch, run, W, K)
        fail_on_flags(sessions, f"the {name} steps of the graph leg")
        out[name] = {"steps": K, "steps_per_s": round(K / (ms * 1e-3), 2),
                     "ms_per_step": round(ms / K, 4), "step_ms": percentiles(per_step)}
    del graphs
    torch.cuda.synchronize()
    return out


def host_gather_leg(torch, wl, qdev, reps=3):
    """KVFetch step 5's host fetch moved three ways, for the F minus S value rows of one
    step of the 32K GQA layer (the rows the step needs from CPU memory):
      zero_copy   the host-row kernel of the decode path, which reads the rows in place
                  (zero-copy loads) and forms their attention terms, with cross-step
                  staging off so every row crosses the link;
      memcpy_runs verkv_gather_rows_memcpy: one hipMemcpyAsync per run of consecutive
                  rows, from the host copy of the fetch list;
      cpu_gather_bulk  the rows gathered by the CPU into a pinned buffer, then one copy;
    and, as the link's ceiling, one contiguous copy of the same byte count."""
    import numpy as np
    from long_context_decode_kvfetch_amd import verkv
    from long_context_decode_kvfetch_amd.runner import Session
    sess = Session(wl, prefetch=False)
    sess.compress()
    for i in range(2):
        sess.step(qdev[i])
    torch.cuda.synchronize()
    res = sess.results_numpy()
    st = sess.state_numpy()
    lists = [F[~h["resident"][F]].astype(np.int32) for F, h in zip(res["fetch"], st)]
    row_bytes = 128 * 2
    nrows = int(sum(x.size for x in lists))
    nbytes = nrows * row_bytes
    cap = sess.shape.caps[0]
    head_bytes = cap * row_bytes
    V = sess.V_host
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # the host-row kernel's time and host bytes averaged over the same steps
    verkv.profile_begin(16 * reps + 16)
    h2d_steps = []
    for i in range(reps):
        sess.step(qdev[2 + i])
        h2d_steps.append(int(sess.results_numpy()["h2d_count"].sum()) * row_bytes)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    zc_ms, zc_n = prof["attend_host"]
    zc_us = zc_ms / zc_n * 1e3
    h2d = int(round(float(np.mean(h2d_steps))))

    def runs_copy():
        off, runs = 0, 0
        for u, x in enumerate(lists):
            runs += verkv.gather_rows_memcpy(V.data_ptr() + u * head_bytes, row_bytes, x,
                                             dst.data_ptr() + off)
            off += x.size * row_bytes
        return runs
    runs_copy()
    torch.cuda.synchronize()
    gpu_ms, cpu_ms = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        e0.record()
        runs = runs_copy()
        e1.record()
        cpu_ms.append((time.perf_counter() - t0) * 1e3)
        torch.cuda.synchronize()
        gpu_ms.append(e0.elapsed_time(e1))
    runs_us = float(np.median(gpu_ms)) * 1e3
    # the rows are identical to the host cache's
    chk = dst[: lists[0].size * row_bytes].view(torch.bfloat16).view(-1, 128).cpu()
    ref = V.view(-1, cap, 128)[0][torch.from_numpy(lists[0]).long()]
    assert torch.equal(chk, ref), "memcpy gather moved the wrong rows"

    bounce = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    bview = bounce.view(torch.bfloat16).view(-1, 128)
    heads = V.view(-1, cap, 128)
    idx_t = [torch.from_numpy(x).long() for x in lists]
    g_ms, c_ms = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        off = 0
        for u, x in enumerate(idx_t):
            torch.index_select(heads[u], 0, x, out=bview[off:off + x.numel()])
            off += x.numel()
        g_ms.append((time.perf_counter() - t0) * 1e3)
        e0.record()
        dst.copy_(bounce, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        c_ms.append(e0.elapsed_time(e1))
    bulk_us = float(np.median(c_ms)) * 1e3
    gather_us = float(np.median(g_ms)) * 1e3
    out = {"workload": "F minus S value rows of one step of the 32K GQA layer (bf16, 256 B per row)",
           "rows": nrows, "bytes": nbytes, "runs": int(runs),
           "mean_run_rows": round(nrows / max(1, runs), 2),
           "zero_copy": {"us": round(zc_us, 1), "GBps": round(h2d / (zc_us * 1e-6) / 1e9, 1),
                         "host_bytes": h2d,
                         "note": "host-row kernel of the decode path, attention terms included, staging off"},
           "memcpy_runs": {"us": round(runs_us, 1), "GBps": round(nbytes / (runs_us * 1e-6) / 1e9, 2),
                           "cpu_issue_ms": round(float(np.median(cpu_ms)), 2)},
           "cpu_gather_bulk": {"us": round(gather_us + bulk_us, 1), "cpu_gather_us": round(gather_us, 1),
                               "copy_us": round(bulk_us, 1), "threads": torch.get_num_threads(),
                               "GBps": round(nbytes / ((gather_us + bulk_us) * 1e-6) / 1e9, 1)},
           "contiguous_copy_ceiling": {"us": round(bulk_us, 1),
                                       "GBps": round(nbytes / (bulk_us * 1e-6) / 1e9, 1)}}
    del sess, dst, bounce
    torch.cuda.empty_cache()
    return out


def sketch2_leg(torch, wls, qdevs, K2, W2):
    """The layer-step with the 2-bit key sketch (64 B per token row instead of 256 B;
    fetched rows are scored from the host keys, so K and V rows cross the host link):
    steps/s over the same rotated layers and the sketch kernel's rate on its own bytes."""
    from long_context_decode_kvfetch_amd import verkv
    from long_context_decode_kvfetch_amd.runner import Session
    L = len(wls)
    sess2 = []
    for wl, qd in zip(wls, qdevs):
        s2 = Session(wl, sketch_2bit=True)
        s2.compress()
        s2.qdev = qd
        sess2.append(s2)
    per_layer = qdevs[0].shape[0]

    def run(i):
        s2 = sess2[i % L]
        s2.step(s2.qdev[(i // L) % per_layer])

    W2 = max(W2, 2 * L)                      # at least two steps per layer: staging primed
    for i in range(W2):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(W2, W2 + K2):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    fail_on_flags(sess2, "the 2-bit sketch leg")
    verkv.profile_begin(8 * 16 + 16)
    for i in range(W2 + K2, W2 + K2 + 16):
        run(i)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    h2d = 0
    for s2 in sess2:
        s2.step(s2.qdev[0])
        h2d += int(s2.results_numpy()["h2d_count"].sum())
    sk_ms, sk_n = prof["sketch_scores"]
    sk_us = sk_ms / sk_n * 1e3
    # per (KV head, token): the 64 B sketch row and r_i (8 B) read (the float64 weights the
    # kernel writes are scratch, 4 x 8 B, not counted)
    sk_bytes = 8 * N_CTX * (64 + R_BYTES)
    host_us = prof["attend_host"][0] / prof["attend_host"][1] * 1e3
    out = {"value": round(K2 / (ms * 1e-3), 2), "unit": "steps/s", "steps": K2,
           "ms_per_step": round(ms / K2, 4),
           "sketch_bytes_per_token_head": 64,
           "sketch_kernel": {"avg_us": round(sk_us, 2), "algorithmic_bytes": sk_bytes,
                             "GBps": round(sk_bytes / (sk_us * 1e-6) / 1e9, 1)},
           "h2d_bytes_per_step": h2d / L * 2 * 128 * 2,
           "host_kernel_avg_us": round(host_us, 1),
           "prefetch_avg_us": round(prof["prefetch"][0] / max(1, prof["prefetch"][1]) * 1e3, 1),
           "note": "the K and V rows of F minus S are read from CPU memory (the sketch is not "
                   "exact); rows the previous step of the layer read are staged, key beside "
                   "value, during the decision kernel and read from the workspace instead "
                   "(h2d_bytes_per_step counts every F minus S row)"}
    del sess2
    torch.cuda.empty_cache()
    return out


EPS_GRID = (0.01, 0.02, 0.05, 0.1, 0.3, 0.5)


def eta_eps_sweep(torch, L, K=32, W=8):
    """The 32K GQA layer-step at resident fractions eta = 1/8, 1/16, 1/32 and tolerances
    eps = 0.01 ... 0.5 (delta = 0.05): steps/s and what crosses the host link, the
    traffic-against-tolerance curve."""
    import copy
    import numpy as np
    from long_context_decode_kvfetch_amd import synth
    from long_context_decode_kvfetch_amd.runner import Session
    base = [synth.gqa_layer(seed=0, n=N_CTX, steps=(K + W + 1 + L - 1) // L + 1, layer=layer)
            for layer in range(L)]
    rows = []
    for eta in (1.0 / 8, 1.0 / 16, 1.0 / 32):
        sess = []
        for wl0 in base:
            wl = copy.copy(wl0)
            wl.eta = eta
            s2 = Session(wl)
            s2.compress()
            s2.qdev = torch.from_numpy(np.ascontiguousarray(wl.queries)).to("cuda")
            sess.append(s2)
        per_layer = sess[0].qdev.shape[0]
        for eps in EPS_GRID:
            def run(i):
                s2 = sess[i % L]
                s2.step(s2.qdev[(i // L) % per_layer], eps=eps)
            for i in range(W):
                run(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(W, W + K):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            fail_on_flags(sess, f"the sweep at eta=1/{round(1 / eta)}, eps={eps}")
            cert = fetched = h2d = nrow = 0
            for s2 in sess:
                s2.step(s2.qdev[0], eps=eps)
                r = s2.results_numpy()
                cert += int(r["certified"].sum())
                fetched += int(r["fetch_count"].sum())
                h2d += int(r["h2d_count"].sum())
                nrow += r["certified"].size
            ntok = L * N_CTX * 8
            rows.append({"eta": eta, "eps": eps, "steps_per_s": round(K / (ms * 1e-3), 1),
                         "rows_certified_without_fetch": cert / nrow,
                         "fetched_fraction_of_cache": fetched / ntok,
                         "h2d_fraction_of_cache": h2d / ntok,
                         "h2d_bytes_per_step": h2d / L * 128 * 2})
            log(f"[bench] sweep eta=1/{round(1 / eta)} eps={eps}: {rows[-1]['steps_per_s']} steps/s, "
                f"F/n {rows[-1]['fetched_fraction_of_cache']:.3f}")
        del sess
        torch.cuda.empty_cache()
    return {"workload": "gqa decode layer-step: 32q/8kv, d=128, n=32768, bf16, exact sketch, "
                        "delta=0.05, layers rotated", "layers": L, "steps": K, "settings": rows}


def decode_36_layers(torch, tokens=16, warm=2, n_layers=36, eta=1.0 / 16, eps_list=(0.05,)):
    """A full decode of one sequence through 36 layers shaped like the 32K GQA layer
    (independent caches, Philox layer word = layer index): every generated token runs
    the 36 layer-steps back to back on one stream, each with its own query rows.  Reports
    tokens/s, milliseconds per layer-step and the bytes that crossed the host link per
    token against the full cache (K and V of 36 layers), for each eps in `eps_list` on
    the same compressed layers (one dict, or a list when several eps are asked for)."""
    import numpy as np
    from long_context_decode_kvfetch_amd import synth
    from long_context_decode_kvfetch_amd.runner import Session
    runs = len(eps_list)
    sess = []
    for layer in range(n_layers):
        wl = synth.gqa_layer(seed=0, n=N_CTX, steps=runs * (tokens + warm + 1), layer=layer, eta=eta)
        s2 = Session(wl)
        s2.compress()
        s2.qdev = torch.from_numpy(np.ascontiguousarray(wl.queries)).to("cuda")
        for sq in wl.seqs:                        # the host copy is pinned; free the arrays
            sq.K = sq.V = None
        sess.append(s2)
        if layer % 6 == 5:
            log(f"[bench] decode36 eta=1/{round(1 / eta)}: {layer + 1} layers compressed")
    torch.cuda.synchronize()
    outs = []
    for k, eps in enumerate(eps_list):
        q0 = k * (tokens + warm + 1)

        def token(t):
            for s2 in sess:
                s2.step(s2.qdev[q0 + t], eps=eps)

        for t in range(warm):
            token(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warm, warm + tokens):
            token(t)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        fail_on_flags(sess, "the 36-layer decode")
        cert = fetched = h2d = nrow = 0
        for s2 in sess:
            s2.step(s2.qdev[q0 + warm + tokens], eps=eps)
            r = s2.results_numpy()
            assert np.all(r["eps_after"] < eps), "a row finished uncertified"
            cert += int(r["certified"].sum())
            fetched += int(r["fetch_count"].sum())
            h2d += int(r["h2d_count"].sum())
            nrow += r["certified"].size
        ntok = n_layers * N_CTX * 8
        full = n_layers * 8 * N_CTX * 128 * 2 * 2                # K and V, bf16, all layers
        resident = sum(int(s2.state.piv_count.sum().item()) for s2 in sess)
        outs.append({"workload": f"{n_layers} layers x (32q/8kv, d=128, n={N_CTX}, bf16, exact sketch), "
                                 f"eta=1/{round(1 / eta)}, eps={eps}, delta=0.05, one sequence",
                     "layers": n_layers, "tokens": tokens, "eta": eta, "eps": eps,
                     "tokens_per_s": round(tokens / (ms * 1e-3), 2),
                     "ms_per_token": round(ms / tokens, 3),
                     "ms_per_layer_step": round(ms / tokens / n_layers, 4),
                     "rows_certified_without_fetch": cert / nrow,
                     "fetched_fraction_of_cache": fetched / ntok,
                     "h2d_bytes_per_token": h2d * 128 * 2,
                     "h2d_fraction_of_full_cache_bytes": h2d * 128 * 2 / full,
                     "full_cache_bytes": full,
                     "resident_pivot_fraction": resident / ntok})
        log(f"[bench] decode36 eta=1/{round(1 / eta)} eps={eps}: {outs[-1]['tokens_per_s']} tokens/s")
    del sess
    torch.cuda.empty_cache()
    return outs[0] if runs == 1 else outs


def long_context_stress(torch, steps=16, warm=2, planted=2048):
    """One 131072-token sequence (32q/8kv, d=128, bf16, eta = 1/32) whose queries align
    with keys planted on tokens the sampler did not keep: PoissonComp runs once, then
    `planted` non-resident tokens per KV head get the heavy-hitter direction and the
    layer is rebuilt (the sample depends only on tau and the seed, so it is the same).
    Steps/s, fetched share and host traffic at eps = 0.05, 0.1, 0.2, 0.3, 0.5."""
    import numpy as np
    from long_context_decode_kvfetch_amd import synth
    from long_context_decode_kvfetch_amd.runner import Session
    n = 131072
    wl = synth.long_context(seed=0, n=n, steps=steps + warm + 1)
    s0 = Session(wl)
    s0.compress()
    resident = np.stack([h["resident"] for h in s0.state_numpy()])
    del s0
    torch.cuda.empty_cache()
    synth.plant_adversarial(wl, resident, planted)
    sess = Session(wl)
    sess.compress()
    qdev = torch.from_numpy(np.ascontiguousarray(wl.queries)).to("cuda")
    for sq in wl.seqs:
        sq.K = sq.V = None
    rows = []
    for eps in (0.05, 0.1, 0.2, 0.3, 0.5):
        for t in range(warm):
            sess.step(qdev[t], eps=eps)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warm, warm + steps):
            sess.step(qdev[t], eps=eps)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        fail_on_flags([sess], f"the long-context leg at eps={eps}")
        sess.step(qdev[warm + steps], eps=eps)
        r = sess.results_numpy()
        assert np.all(r["eps_after"] < eps), "a row finished uncertified"
        ntok = n * 8
        rows.append({"eps": eps, "steps_per_s": round(steps / (ms * 1e-3), 2),
                     "ms_per_step": round(ms / steps, 3),
                     "rows_certified_without_fetch": float(r["certified"].mean()),
                     "fetched_fraction_of_cache": int(r["fetch_count"].sum()) / ntok,
                     "h2d_fraction_of_cache": int(r["h2d_count"].sum()) / ntok,
                     "h2d_bytes_per_step": int(r["h2d_count"].sum()) * 128 * 2})
        log(f"[bench] long context eps={eps}: {rows[-1]['steps_per_s']} steps/s, "
            f"F-S/n {rows[-1]['h2d_fraction_of_cache']:.3f}")
    piv = int(sess.state.piv_count.sum().item())
    del sess
    torch.cuda.empty_cache()
    return {"workload": f"one sequence n={n}, 32q/8kv, d=128, bf16, exact sketch, eta=1/32, "
                        f"H=4 sink+128 local, {planted} keys per KV head planted on non-resident "
                        "tokens, delta=0.05", "pivot_rows": piv,
            "pivot_bytes_per_step": piv * 128 * 2 * 2, "steps": steps, "settings": rows}


def calib_copy(torch):
    """A kernel of known traffic for scaling FETCH_SIZE / WRITE_SIZE: an elementwise copy
    that reads and writes 256 MiB once per launch, three launches."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(steps):
    """The oracle (as it stands) on the benchmark's workload: one layer, `steps` decode
    steps of the 32K GQA layer, with every thread pool of the process limited to one
    thread and with the default threads; plus one step of the single-head workload
    (n = 4096, fp32, G = 8).  Prefill is excluded."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from long_context_decode_kvfetch_amd import synth
    from oracle import api as oapi
    wl = synth.gqa_layer(seed=0, n=N_CTX, steps=steps, layer=0)
    s = wl.seqs[0]
    comp = oapi.compress_sequence(s.tau, wl.n_sink, wl.n_local, wl.eta, 0, 0, wl.seed)
    w1 = synth.single_head(0)
    s1 = w1.seqs[0]
    c1 = oapi.compress_sequence(s1.tau, w1.n_sink, w1.n_local, w1.eta, 0, 0, w1.seed)

    def run():
        t0 = time.perf_counter()
        for st in range(steps):
            oapi.decode_sequence(s.K, s.V, comp, wl.queries[st, 0], wl.group, wl.kappa, wl.eps,
                                 wl.delta)
        t1 = time.perf_counter()
        oapi.decode_sequence(s1.K, s1.V, c1, w1.queries[0, 0], w1.group, w1.kappa, w1.eps, w1.delta)
        return t1 - t0, time.perf_counter() - t1

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    dt_all, dt1_all = run()
    with threadpool_limits(1):
        dt_one, dt1_one = run()

    # bounded samples of the other shapes, default threads: the 16-sequence batch by one
    # sequence of its mean length (lengths uniform in [8K, 64K]), and one step of the 131K
    # stress shape (eta = 1/32, no planted keys)
    def one_step(wl_):
        sq = wl_.seqs[0]
        cp = oapi.compress_sequence(sq.tau, wl_.n_sink, wl_.n_local, wl_.eta, 0, 0, wl_.seed)
        t0 = time.perf_counter()
        oapi.decode_sequence(sq.K, sq.V, cp, wl_.queries[0, 0], wl_.group, wl_.kappa, wl_.eps, wl_.delta)
        return time.perf_counter() - t0
    n_mean = (8192 + 65536) // 2
    dt_b = one_step(synth.gqa_layer(seed=0, n=n_mean, steps=1, layer=0))
    del wl, s, comp
    dt_l = one_step(synth.long_context(seed=0, n=131072, steps=1, eps=0.05))
    return {"value": steps / dt_all, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} decode steps of one 32K GQA layer (32q/8kv, n={N_CTX}, bf16 values "
                      f"in float64, eta=1/16), prefill excluded: {dt_all:.1f} s with the default "
                      f"{threads} threads, {dt_one:.1f} s on one thread",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": steps / dt_one, "unit": "steps/s", "cores": 1},
            "single_head_n4096_ms": {"default_threads": round(dt1_all * 1e3, 1),
                                     "one_thread": round(dt1_one * 1e3, 1)},
            "batch16_step_s": {"value": round(16 * dt_b, 2),
                               "sample": f"one step of one {n_mean}-token sequence (the batch's mean "
                                         f"length) took {dt_b:.2f} s; x 16 sequences"},
            "long_context_131k_step_s": {"value": round(dt_l, 2),
                                         "sample": "one step of the 131072-token layer, eta=1/32, "
                                                   "eps=0.05, no planted keys"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the KVFetch path shards by sequence and KV head with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from long_context_decode_kvfetch_amd import synth, verkv
    from long_context_decode_kvfetch_amd.runner import Session

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        print(json.dumps({"sweep": eta_eps_sweep(torch, args.layers)}))
        return
    if args.decode36:
        print(json.dumps({"decode_36_layers": decode_36_layers(torch)}))
        return
    if args.decode36_grid:
        grid = []
        for eta in (1.0 / 8, 1.0 / 16, 1.0 / 32):
            grid += decode_36_layers(torch, tokens=8, eta=eta, eps_list=(0.02, 0.05, 0.1))
        print(json.dumps({"decode_36_layers_grid": grid}))
        return
    if args.long_context:
        print(json.dumps({"long_context": long_context_stress(torch)}))
        return
    if args.pivot_only:
        if args.calib_copy:
            calib_copy(torch)
        log("[bench] pivotal stream at the 16-sequence batch")
        print(json.dumps({"pivotal_stream": pivotal_stream(torch)}))
        return
    K, W, L = args.steps, args.warmup, args.layers
    total = K + W + args.profile_steps + 1
    per_layer = (total + L - 1) // L + 2
    log(f"[bench] generating {L} layers (n={N_CTX}, 32q/8kv, bf16)")
    sessions = []
    for layer in range(L):
        wl = synth.gqa_layer(seed=0, n=N_CTX, steps=per_layer, layer=layer)
        sess = Session(wl)
        sess.compress()
        sess.qdev = torch.from_numpy(np.ascontiguousarray(wl.queries[:, :])).to("cuda")
        sessions.append(sess)
        log(f"[bench] layer {layer} compressed, max pivots {sess.max_pivots}, cap {sess.cap}")
    # two steps per layer before any counted step, as every layer of a running decode has
    # had: the first leaves a staging plan for the whole area (nothing is staged yet), the
    # second copies it; from then on a step copies only the rows new to the list
    for prime in (2, 1):
        for sess in sessions:
            sess.step(sess.qdev[per_layer - prime])
    torch.cuda.synchronize()

    def run(step_index):
        sess = sessions[step_index % L]
        sess.step(sess.qdev[(step_index // L) % per_layer])
        return sess

    if args.calib_copy:
        calib_copy(torch)

    for i in range(W):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_ms, per_step = timed(torch, run, W, K)
    wall = time.perf_counter() - t0
    ms_per_step = ev_ms / K
    fail_on_flags(sessions, "the timed steps")
    log(f"[bench] {K} steps: {wall * 1e3:.1f} ms wall, {ev_ms:.1f} ms events")

    # per-step statistics over one pass of every layer
    cert, fetched, h2d, staged, rows, n_tok = 0, 0, 0, 0, 0, 0
    for sess in sessions:
        sess.step(sess.qdev[0])
        r = sess.results_numpy()
        cert += int(r["certified"].sum())
        fetched += int(r["fetch_count"].sum())
        h2d += int(r["h2d_count"].sum())
        staged += sess.staged_rows()          # of those, rows served by the staging area
        rows += r["certified"].size
        n_tok += N_CTX * sess.shape.n_kv_heads
        assert np.all(r["eps_after"] < sess.wl.eps), "a row finished uncertified"
    # exact sketch: only the value rows of F minus S are read (256 B each); the staged ones
    # come from the workspace, the rest over the host link
    h2d_bytes_step = h2d / L * 128 * 2
    link_bytes_step = (h2d - staged) / L * 128 * 2

    # kernel durations with HIP events around every launch of the profiled steps
    P = args.profile_steps
    verkv.profile_begin(8 * P + 16)
    for i in range(W + K, W + K + P):
        run(i)
    torch.cuda.synchronize()
    prof = verkv.profile_report()
    verkv.profile_end()
    fail_on_flags(sessions, "the profiled steps")
    piv_rows = sum(int(s.state.piv_count.sum().item()) for s in sessions) / L
    piv_bytes = piv_rows * PIVOT_ROW_BYTES
    tok_heads = 8 * N_CTX
    sk_bytes = sketch_bytes(tok_heads)
    kern = {}
    for name, (ms, cnt) in prof.items():
        if cnt:
            kern[name] = {"avg_us": ms / cnt * 1e3, "launches": cnt}
    sk = kern["sketch_scores"]
    sk["algorithmic_bytes"] = sk_bytes
    sk["GBps"] = sk_bytes / (sk["avg_us"] * 1e-6) / 1e9
    # the float64 sketch weights the kernel leaves for the decision kernels: scratch
    sk["scratch_write_bytes"] = tok_heads * WHAT_SCRATCH_BYTES
    kern["attend_pivots"]["algorithmic_bytes"] = piv_bytes
    kern["attend_pivots"]["GBps"] = piv_bytes / (kern["attend_pivots"]["avg_us"] * 1e-6) / 1e9
    kern["attend_host"]["host_bytes"] = h2d_bytes_step
    kern["attend_host"]["GBps"] = h2d_bytes_step / (kern["attend_host"]["avg_us"] * 1e-6) / 1e9
    kern["attend_host"]["link_bytes"] = link_bytes_step
    kern["attend_host"]["link_GBps"] = link_bytes_step / (kern["attend_host"]["avg_us"] * 1e-6) / 1e9
    # The roofline kernel is the sketch scoring pass: the HBM stream on the step's
    # critical path.  The host-row kernel is bound by the host link (reported against
    # the pinned-copy rate below); the resident-pivot and eps_after kernels run on the
    # library's second stream in the shadow of the host rows, so their durations there
    # include sharing the CUs with it and do not bound the step.
    dom = "sketch_scores"
    for k in ("attend_pivots", "eps_after", "pivot_coef"):
        if k in kern:
            kern[k]["overlapped_with"] = "attend_host"
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(kern[dom]["GBps"], 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern[dom]["GBps"] / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic(dom) if dom in KERNEL_SOURCES else None,
            "algorithmic_bytes": kern[dom]["algorithmic_bytes"],
            "bytes_per_unit": "264 B per (KV head, token): bf16 key row + float64 r",
            "units_per_launch": tok_heads}
    step_bytes = step_algorithmic_bytes(tok_heads, piv_rows)
    h2d_peak = h2d_bandwidth(torch)
    resolved = None
    if not args.no_resolved:
        log("[bench] re-solved reading of eqs. (9)-(10) on the same layers")
        resolved = resolved_leg(torch, sessions, K=min(K, 64), W=min(W, 8))
    nofetch = None
    if not args.no_nofetch:
        log("[bench] no-fetch control: uniform scores, eps = 0.2")
        nofetch = no_fetch_leg(torch, L)
    staging = None
    if not args.no_staging:
        log("[bench] staging slots per KV head: sweep")
        staging = staging_leg(torch, [s.wl for s in sessions], [s.qdev for s in sessions],
                              K=min(K, 64), W=min(W, 8))
    graph = None
    if not args.no_graph:
        log("[bench] one HIP graph per layer-step, replayed")
        graph = graph_leg(torch, sessions, K=min(K, 64), W=min(W, 8))
    gather = None
    if not args.no_gather:
        log("[bench] host fetch: zero-copy kernel against memcpy per run")
        gather = host_gather_leg(torch, sessions[0].wl, sessions[0].qdev)
    sk2 = None
    if not args.no_2bit:
        log("[bench] 2-bit sketch: the same layers, rebuilt")
        wls = [sess.wl for sess in sessions]
        qdevs = [sess.qdev for sess in sessions]
        sessions.clear()
        torch.cuda.empty_cache()
        sk2 = sketch2_leg(torch, wls, qdevs, K2=min(K, 64), W2=min(W, 8))
    sessions.clear()
    torch.cuda.empty_cache()
    piv = None
    if not args.no_pivot_batch:
        log("[bench] 16-sequence batch: pivotal stream, then eps = 0.05")
        piv = pivotal_stream(torch)
    dec36 = None
    if not args.no_decode36:
        log("[bench] 36-layer decode")
        dec36 = decode_36_layers(torch)
    longc = None
    if not args.no_long_context:
        log("[bench] long-context stress")
        longc = long_context_stress(torch)

    out = {
        "metric": "certified decode steps/s at 32K ctx, eta=1/16; achieved HBM GB/s vs peak",
        "value": round(K / (ev_ms * 1e-3), 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64+f32",
        "data": "synthetic",
        "config": {"workload": "gqa decode layer-step: 32q/8kv heads, d=128, n=32768, bf16 "
                               "cache in pinned host memory, exact sketch, eta=1/16, "
                               "H=4 sink+128 local, eps=0.05, delta=0.05, 1% planted heavy "
                               "hitters, tau~Beta(0.3,3)",
                   "layers_rotated": L, "seq_len": N_CTX, "batch": 1},
        "roofline": roof,
        "step_ms": percentiles(per_step),
        "whole_step": {"algorithmic_bytes": int(step_bytes),
                       "GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                       "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "note": "sketch stream + pivotal stream + bitmasks per layer-step over "
                               "the step time; the host rows of F minus S are counted apart "
                               "(step_stats.h2d_bytes_per_step)"},
        "pivotal_stream": piv,
        "no_fetch": nofetch,
        "host_fetch_variants": gather,
        "graph_replay": graph,
        "staging_slots": staging,
        "resolved_reading": resolved,
        "sketch_2bit": sk2,
        "decode_36_layers": dec36,
        "long_context": longc,
        "cpu_baseline": None,
        "step_stats": {"rows_certified_without_fetch": cert / rows,
                       "fetched_fraction_of_cache": fetched / n_tok,
                       "h2d_fraction_of_cache": h2d / n_tok,
                       "h2d_bytes_per_step": h2d_bytes_step,
                       "h2d_GBps_per_step": h2d_bytes_step / (ms_per_step * 1e-3) / 1e9,
                       "staged_bytes_per_step": h2d_bytes_step - link_bytes_step,
                       "host_link_bytes_per_step": link_bytes_step,
                       "host_link_GBps_per_step": link_bytes_step / (ms_per_step * 1e-3) / 1e9,
                       "pinned_h2d_copy_GBps": round(h2d_peak, 1),
                       "wall_ms_per_step": wall * 1e3 / K},
        "kernels": kern,
    }
    if not args.no_cpu:
        log(f"[bench] cpu baseline: oracle, {args.cpu_steps} steps")
        out["cpu_baseline"] = cpu_baseline(args.cpu_steps)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
