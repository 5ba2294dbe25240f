"""Runs a synthetic workload through the library: uploads the cache, compresses it
and executes decode steps.  Used by the tests, the benchmark and the smoke check.

Exact-sketch mode: the device-resident sketch is the key cache itself (the setting of
Theorem 2 on the picx.dev summary page).  The complete K/V cache lives in pinned host
memory; only H u S and the sketch are on the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

from . import verkv
from .synth import Workload


def _cat(arrs, caps=None):
    """Sequence-major concatenation of per-sequence [Hkv][n][...] arrays, each padded with
    zeros to its capacity along the token axis."""
    if caps is None:
        return np.concatenate([a.reshape(-1) for a in arrs])
    out = []
    for a, c in zip(arrs, caps):
        pad = [(0, 0), (0, int(c) - a.shape[1])] + [(0, 0)] * (a.ndim - 2)
        out.append(np.pad(a, pad).reshape(-1))
    return np.concatenate(out)


class Session:
    """One layer of a workload, compressed on the GPU, ready for decode steps."""

    def __init__(self, wl: Workload, cap: int | None = None, device: str = "cuda",
                 host_pinned: bool = True, seed: int | None = None, sketch_exact: bool = True,
                 prefetch: bool = True, sketch_2bit: bool = False, grow: int = 0,
                 stage_slots: int = 0):
        """grow: token slots reserved past each sequence's length for append();
        stage_slots: rows per KV head of the cross-step staging (0: the library's default)."""
        self.wl = wl
        self.device = device
        lens = [s.n for s in wl.seqs]
        caps = [n + int(grow) for n in lens] if grow else None
        self.shape = verkv.LayerShape(lens, wl.n_kv_heads, wl.group, wl.n_sink, wl.n_local,
                                      wl.kv_dtype, wl.layer, caps, stage_slots)
        dt = self.shape.torch_dtype
        K = torch.from_numpy(_cat([s.K for s in wl.seqs], caps)).to(dt)
        V = torch.from_numpy(_cat([s.V for s in wl.seqs], caps)).to(dt)
        if host_pinned:
            self.K_host = torch.empty(K.shape, dtype=dt, pin_memory=True)
            self.V_host = torch.empty(V.shape, dtype=dt, pin_memory=True)
            self.K_host.copy_(K)
            self.V_host.copy_(V)
        else:                                   # whole cache on the device (tests only)
            self.K_host = K.to(device)
            self.V_host = V.to(device)
        if sketch_2bit:
            # the 2-bit sketch of the keys (64 B per token row), quantised on the device
            # from the host cache; fetched rows are then scored from the host keys
            nbytes = self.shape.total_slots * self.shape.n_kv_heads * verkv.SKETCH2_ROW_BYTES
            self.sketch = torch.empty(nbytes, dtype=torch.uint8, device=device)
            verkv.quantize_sketch(self.shape, self.K_host, self.sketch)
            sketch_exact = False
        else:
            self.sketch = K.to(device)          # exact sketch: the keys, device resident
        self.tau = torch.from_numpy(_cat([s.tau for s in wl.seqs], caps).astype(np.float32)).to(device)
        self.cap = int(cap) if cap else verkv.default_cap(self.shape, wl.eta)
        self.state = verkv.LayerState(self.shape, self.cap, self.sketch, device, sketch_exact,
                                      v_host=self.V_host if (host_pinned and prefetch) else None,
                                      k_host=self.K_host if (host_pinned and prefetch and not sketch_exact) else None,
                                      sketch_format=verkv.SKETCH_2BIT if sketch_2bit else verkv.SKETCH_ROWS)
        self.cws = verkv.workspace(self.shape.compress_workspace_bytes(), device)
        self.dws = verkv.workspace(self.shape.decode_workspace_bytes(self.cap), device)
        self.out = verkv.StepBuffers(self.shape, fetch_cap=max(self.shape.caps), device=device)
        self.seed = wl.seed if seed is None else seed
        self.max_pivots = None
        self.sketch_2bit = sketch_2bit
        self.aws = None
        self.astatus = None

    def compress(self, stream=None):
        self.max_pivots = verkv.compress(self.shape, self.tau, self.K_host, self.V_host,
                                         self.wl.eta, self.seed, self.state, self.cws, stream)
        return self.max_pivots

    def _slot(self, b: int, g: int, i: int) -> int:
        """Flat token slot of (sequence b, KV head g, token i) in the capacity-strided arrays."""
        caps = self.shape.caps
        return self.shape.n_kv_heads * sum(caps[:b]) + g * caps[b] + i

    def append(self, k_rows: np.ndarray, v_rows: np.ndarray, tau_new: np.ndarray, stream=None):
        """Append one token to every sequence: k_rows, v_rows [B][Hkv][128] (values the cache
        dtype holds exactly), tau_new [B][Hkv].  Writes the rows into the host cache and the
        exact sketch, the scores into tau, calls verkv_append and grows the shape.  Returns
        the status word (a device tensor; nonzero means nothing changed)."""
        if self.max_pivots is None:
            raise RuntimeError("Session.append before compress()")
        if self.sketch_2bit:
            raise NotImplementedError("append with a 2-bit sketch needs the new rows re-quantised")
        if self.aws is None:
            self.aws = verkv.workspace(self.shape.append_workspace_bytes(self.cap), self.device)
            self.astatus = torch.zeros(1, dtype=torch.int32, device=self.device)
        dt = self.shape.torch_dtype
        hkv = self.shape.n_kv_heads
        idx = [self._slot(b, g, n) for b, n in enumerate(self.shape.seq_lens) for g in range(hkv)]
        kr = torch.from_numpy(np.ascontiguousarray(k_rows, dtype=np.float32).reshape(-1, 128)).to(dt)
        vr = torch.from_numpy(np.ascontiguousarray(v_rows, dtype=np.float32).reshape(-1, 128)).to(dt)
        it = torch.tensor(idx, dtype=torch.long)
        self.K_host.view(-1, 128)[it] = kr.to(self.K_host.device)
        self.V_host.view(-1, 128)[it] = vr.to(self.V_host.device)
        itd = it.to(self.device)
        if not self.sketch_2bit:
            self.sketch.view(-1, 128)[itd] = kr.to(self.device)
        self.tau[itd] = torch.from_numpy(np.ascontiguousarray(tau_new, dtype=np.float32).reshape(-1)).to(self.device)
        verkv.append(self.shape, self.state, self.tau, self.K_host, self.V_host, self.seed,
                     self.astatus, self.aws, stream)
        self.shape = self.shape.grown(1)
        return self.astatus

    def queries(self, step: int) -> torch.Tensor:
        """Query rows of one step as a device tensor [B][Hq][128] (float32)."""
        return torch.from_numpy(np.ascontiguousarray(self.wl.queries[step])).to(self.device)

    def step(self, q: torch.Tensor, kappa=None, eps=None, delta=None, stream=None,
             out: verkv.StepBuffers | None = None, resolved: bool = False):
        if self.max_pivots is None:
            raise RuntimeError("Session.step before compress(): the pivot state is not written")
        out = out or self.out
        wl = self.wl
        verkv.decode_step(self.shape, self.state, q, wl.kappa if kappa is None else kappa,
                          wl.eps if eps is None else eps, wl.delta if delta is None else delta,
                          out, self.dws, stream, resolved=resolved)
        verkv.refine(self.shape, self.state, q, self.K_host, self.V_host, out, self.dws, stream)
        return out

    def staged_rows(self) -> int:
        """Rows of the last step's F minus S taken from the staging area, not the host link."""
        return verkv.staged_rows(self.shape, self.cap, self.dws)

    # ---------------------------------------------------------------- host-side views
    def state_numpy(self):
        """r, resident mask, pivot lists per (sequence, KV head)."""
        torch.cuda.synchronize()
        r = self.state.r.cpu().numpy()
        res = self.state.resident.cpu().numpy().view(np.uint32)
        cnt = self.state.piv_count.cpu().numpy()
        pidx = self.state.piv_idx.view(-1, self.cap).cpu().numpy()
        out = []
        roff, woff = 0, 0
        for b, (n, c) in enumerate(zip(self.shape.seq_lens, self.shape.caps)):
            W = (c + 31) // 32
            for g in range(self.shape.n_kv_heads):
                u = b * self.shape.n_kv_heads + g
                bits = np.unpackbits(res[woff + g * W: woff + (g + 1) * W].view(np.uint8),
                                     bitorder="little")[:n].astype(bool)
                out.append(dict(r=r[roff + g * c: roff + g * c + n], resident=bits,
                                piv_idx=pidx[u, :min(int(cnt[u]), self.cap)], piv_count=int(cnt[u])))
            roff += self.shape.n_kv_heads * c
            woff += self.shape.n_kv_heads * W
        return out

    def results_numpy(self, out: verkv.StepBuffers | None = None):
        out = out or self.out
        torch.cuda.synchronize()
        rows = self.shape.batch * self.shape.n_q_heads
        res = {k: getattr(out, k).cpu().numpy() for k in
               ("m_hat", "d_sketch", "beta_star", "eps_hat", "certified", "kstar", "eps_after",
                "d_hat", "lse", "fetch_count", "h2d_count")}
        res["o"] = out.o.view(rows, -1).cpu().numpy()
        res["n_hat"] = out.n_hat.view(rows, -1).cpu().numpy()
        res["fetch"] = out.fetch_lists(self.shape)
        return res
