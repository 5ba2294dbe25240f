"""Seeded synthetic inputs for the KVFetch decode path.

This module only draws data.  It holds none of the method's arithmetic (no
water-filling, no sampling, no estimator), so that both the fp64 oracle and the
HIP path can take their inputs from it without sharing any code with each other.

The workloads of "Verify Before You Fetch" (RULER and LOFT on BF16 models, page
"picx.dev summary", section "Experimental Setup") are not available here; these
generators stand in for them with the same shapes: Qwen3-4B-shaped GQA (32 query
heads over 8 KV heads, head_dim 128), 32K and 128K contexts, bf16 caches.

Every array is numpy.  Keys and values that the path stores as bf16 are returned
as float32 arrays whose every element is exactly representable in bf16 (rounded
to nearest-even once, here), so the oracle and the GPU see identical numbers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); result is float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    # NaN/Inf do not occur in these generators (finite normal draws).
    return out.reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Sequence:
    """One sequence of one layer: cache, importance scores and planted structure."""
    n: int
    K: np.ndarray            # [Hkv][n][d] float32 (bf16-exact if kv_dtype == "bf16")
    V: np.ndarray            # [Hkv][n][d]
    tau: np.ndarray          # [Hkv][n] float32 in [0, 1]
    u: np.ndarray            # [Hkv][d] planted unit directions
    heavy: list              # per KV head: sorted int array of planted heavy-hitter positions


@dataclass
class Workload:
    name: str
    n_kv_heads: int
    group: int               # query rows per KV head (GQA group size)
    kv_dtype: str            # "bf16" or "f32"
    n_sink: int
    n_local: int
    eta: float
    kappa: float             # multiplier on the shrinkage bias term (1 = the paper's estimator)
    eps: float
    delta: float
    seed: int
    layer: int
    seqs: list               # list[Sequence]
    queries: np.ndarray = field(default=None)   # [steps][B][Hq][d] float32

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def batch(self) -> int:
        return len(self.seqs)


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    v = rng.standard_normal(d)
    return (v / np.linalg.norm(v)).astype(np.float64)


def _plant(rng, K, u, count, n_sink, n_local, scale):
    """Add scale*u to `count` keys drawn uniformly among non-forced positions."""
    n = K.shape[0]
    pool = np.arange(n_sink, n - n_local)
    pos = np.sort(rng.choice(pool, size=min(count, pool.size), replace=False))
    K[pos] += (scale * u).astype(np.float32)
    return pos


def _queries(rng, u_per_kv, group, steps, noise_var):
    """q = u_{g(h)} + N(0, noise_var I), one row per query head, per step."""
    hkv, d = u_per_kv.shape
    base = np.repeat(u_per_kv, group, axis=0)                   # [Hq][d]
    noise = rng.standard_normal((steps, hkv * group, d)) * math.sqrt(noise_var)
    return (base[None] + noise).astype(np.float32)


def _gqa_sequence(rng, n, hkv, d, kv_dtype, hh_frac, n_sink, n_local, tau_kind):
    K = rng.standard_normal((hkv, n, d), dtype=np.float32)
    V = rng.standard_normal((hkv, n, d), dtype=np.float32)
    us = np.stack([_unit(rng, d) for _ in range(hkv)])
    heavy = []
    for g in range(hkv):
        cnt = int(round(hh_frac * n))
        heavy.append(_plant(rng, K[g], us[g], cnt, n_sink, n_local, 4.0 * math.sqrt(d)))
    if tau_kind == "beta":
        tau = rng.beta(0.3, 3.0, size=(hkv, n)).astype(np.float32)
    elif tau_kind == "uniform":
        tau = rng.random((hkv, n)).astype(np.float32)
    else:
        raise ValueError(tau_kind)
    if kv_dtype == "bf16":
        K = round_bf16(K)
        V = round_bf16(V)
    return Sequence(n=n, K=K, V=V, tau=tau, u=us, heavy=heavy)


def single_head(seed: int = 0, n: int = 4096) -> Workload:
    """Single head, single layer: n=4096, d=128, fp32 K/V ~ N(0,1), 16 planted
    heavy-hitter keys (+4*sqrt(d) along a random unit direction u), one decode
    step with 8 query rows each = u + N(0, 0.5 I); tau = Zipf(1.1) profile
    rho^-1.1 over a random permutation rho of 1..n; H = 4 sink + 64 local;
    eta = 1/8, kappa = 1, eps = 0.05, delta = 0.05."""
    rng = np.random.default_rng(seed)
    d = HEAD_DIM
    n_sink, n_local = 4, 64
    K = rng.standard_normal((1, n, d), dtype=np.float32)
    V = rng.standard_normal((1, n, d), dtype=np.float32)
    u = _unit(rng, d)
    heavy = _plant(rng, K[0], u, 16, n_sink, n_local, 4.0 * math.sqrt(d))
    rho = rng.permutation(n) + 1
    tau = (rho.astype(np.float64) ** -1.1).astype(np.float32)[None]
    seq = Sequence(n=n, K=K, V=V, tau=tau, u=u[None], heavy=[heavy])
    wl = Workload(name=f"single-head n={n} d=128 G=8 fp32 eta=1/8", n_kv_heads=1, group=8,
                  kv_dtype="f32", n_sink=n_sink, n_local=n_local, eta=1.0 / 8, kappa=1.0,
                  eps=0.05, delta=0.05, seed=seed, layer=0, seqs=[seq])
    wl.queries = _queries(rng, u[None], 8, 1, 0.5)[:, None]
    return wl


def gqa_layer(seed: int = 0, n: int = 32768, steps: int = 256, eta: float = 1.0 / 16,
              eps: float = 0.05, delta: float = 0.05, layer: int = 0, hkv: int = 8,
              group: int = 4, n_sink: int = 4, n_local: int = 128,
              tau_kind: str = "beta", hh_frac: float = 0.01, kv_dtype: str = "bf16") -> Workload:
    """Qwen3-4B-shaped decode, one layer: 32 Q / 8 KV heads, d=128, bf16 K/V ~ N(0,1)
    with 1% planted heavy hitters per KV head, tau ~ Beta(0.3, 3), H = 4 sink +
    128 local, eta = 1/16, one query token per step (q_h = u_{g(h)} + N(0, 0.5 I))."""
    rng = np.random.default_rng([seed, layer])
    seq = _gqa_sequence(rng, n, hkv, HEAD_DIM, kv_dtype, hh_frac, n_sink, n_local, tau_kind)
    wl = Workload(name=f"gqa {hkv * group}q/{hkv}kv n={n} d=128 {kv_dtype} eta=1/{round(1 / eta)}",
                  n_kv_heads=hkv, group=group, kv_dtype=kv_dtype, n_sink=n_sink, n_local=n_local,
                  eta=eta, kappa=1.0, eps=eps, delta=delta, seed=seed, layer=layer, seqs=[seq])
    wl.queries = _queries(rng, seq.u, group, steps, 0.5)[:, None]
    return wl


def ragged_batch(seed: int = 0, batch: int = 16, n_min: int = 8192, n_max: int = 65536,
                 steps: int = 1, eta: float = 1.0 / 16, eps: float = 0.05, delta: float = 0.05,
                 hkv: int = 8, group: int = 4, n_sink: int = 4, n_local: int = 128) -> Workload:
    """Batched decode: `batch` sequences with lengths uniform in [n_min, n_max],
    32 Q / 8 KV heads, d=128, bf16, eta = 1/16; sequence b uses Philox stream id b."""
    rng = np.random.default_rng([seed, 4242])
    lens = rng.integers(n_min, n_max + 1, size=batch)
    seqs = [_gqa_sequence(rng, int(nb), hkv, HEAD_DIM, "bf16", 0.01, n_sink, n_local, "beta")
            for nb in lens]
    wl = Workload(name=f"ragged batch B={batch} n in [{n_min},{n_max}] 32q/8kv bf16 eta=1/16",
                  n_kv_heads=hkv, group=group, kv_dtype="bf16", n_sink=n_sink, n_local=n_local,
                  eta=eta, kappa=1.0, eps=eps, delta=delta, seed=seed, layer=0, seqs=seqs)
    qs = [_queries(rng, s.u, group, steps, 0.5) for s in seqs]      # each [steps][Hq][d]
    wl.queries = np.stack(qs, axis=1)
    return wl


def long_context(seed: int = 0, n: int = 131072, steps: int = 1, eps: float = 0.1,
                 delta: float = 0.05) -> Workload:
    """Long-context stress: one sequence, n = 131072, 32 Q / 8 KV heads, d=128, bf16,
    eta = 1/32.  The adversarial keys are planted afterwards by `plant_adversarial`,
    which needs the resident mask that PoissonComp drew."""
    wl = gqa_layer(seed=seed, n=n, steps=steps, eta=1.0 / 32, eps=eps, delta=delta)
    wl.name = f"long-context n={n} 32q/8kv bf16 eta=1/32"
    return wl


def plant_adversarial(wl: Workload, resident: np.ndarray, count: int, seed: int = 1) -> None:
    """Plant +4*sqrt(d)*u_g on `count` non-resident tokens per KV head, in place.

    `resident` is a boolean [Hkv][n] mask of the tokens the sampler kept (passed
    in: this module draws no part of the method's randomness).  Queries aligned
    with u_g then weight tokens that are not on the GPU."""
    rng = np.random.default_rng([seed, 777])
    seq = wl.seqs[0]
    d = seq.K.shape[2]
    for g in range(wl.n_kv_heads):
        pool = np.flatnonzero(~resident[g])
        pool = pool[(pool >= wl.n_sink) & (pool < seq.n - wl.n_local)]
        pos = np.sort(rng.choice(pool, size=min(count, pool.size), replace=False))
        add = (4.0 * math.sqrt(d) * seq.u[g]).astype(np.float32)
        vals = seq.K[g, pos] + add
        seq.K[g, pos] = round_bf16(vals) if wl.kv_dtype == "bf16" else vals
        seq.heavy[g] = np.union1d(seq.heavy[g], pos)


def tiny(seed: int, n: int, hkv: int = 1, group: int = 2, n_sink: int = 1, n_local: int = 1,
         eta: float = 0.5, kv_dtype: str = "f32", tau_kind: str = "uniform",
         logit_scale: float = 1.0) -> Workload:
    """Small random instance for brute-force checks (n up to a few dozen)."""
    rng = np.random.default_rng([seed, n, 99])
    d = HEAD_DIM
    K = (rng.standard_normal((hkv, n, d)) * logit_scale).astype(np.float32)
    V = rng.standard_normal((hkv, n, d), dtype=np.float32)
    if tau_kind == "uniform":
        tau = rng.random((hkv, n)).astype(np.float32)
    else:
        tau = rng.beta(0.3, 3.0, size=(hkv, n)).astype(np.float32)
    if kv_dtype == "bf16":
        K, V = round_bf16(K), round_bf16(V)
    us = np.stack([_unit(rng, d) for _ in range(hkv)])
    seq = Sequence(n=n, K=K, V=V, tau=tau, u=us, heavy=[np.zeros(0, np.int64)] * hkv)
    wl = Workload(name=f"tiny n={n}", n_kv_heads=hkv, group=group, kv_dtype=kv_dtype,
                  n_sink=n_sink, n_local=n_local, eta=eta, kappa=1.0, eps=0.05, delta=0.05,
                  seed=seed, layer=0, seqs=[seq])
    wl.queries = (rng.standard_normal((1, 1, hkv * group, d))).astype(np.float32)
    return wl
