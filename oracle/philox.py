"""Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), written from the
published definition.  Test infrastructure for the oracle only.

The summary page ("Methodology", PoissonComp) asks only that the Bernoulli draws
Z_i be independent; a counter-based generator makes every draw a pure function of
(seed, token, head, layer, sequence), so the CPU and the GPU can reproduce the
same sample independently.

A Philox4x32 round maps a 128-bit counter (c0, c1, c2, c3) under a 64-bit key
(k0, k1) with two 32x32->64 multiplications:
    (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2
    (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
and the key is advanced by the Weyl constants between rounds.  Ten rounds.
"""
import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF
ROUNDS = 10


def philox4x32(c0, c1, c2, c3, k0, k1, rounds=ROUNDS):
    """Vectorised Philox4x32-R; every argument is an array-like of uint32 values
    (broadcast together).  Returns four uint64 arrays holding 32-bit words."""
    u64 = np.uint64
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(*(np.asarray(x, dtype=u64)
                                                    for x in (c0, c1, c2, c3, k0, k1)))
    c0, c1, c2, c3, k0, k1 = (x.copy() for x in (c0, c1, c2, c3, k0, k1))
    m = u64(MASK32)
    for rnd in range(rounds):
        if rnd:
            k0 = (k0 + u64(W0)) & m
            k1 = (k1 + u64(W1)) & m
        p0 = u64(M0) * c0          # < 2^64: exact in uint64
        p1 = u64(M1) * c2
        hi0, lo0 = p0 >> u64(32), p0 & m
        hi1, lo1 = p1 >> u64(32), p1 & m
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def seed_key(seed: int):
    """Key words from a 64-bit seed: (seed mod 2^32, seed >> 32)."""
    seed = int(seed) & ((1 << 64) - 1)
    return seed & MASK32, (seed >> 32) & MASK32


def uniform53(token, kv_head: int, layer: int, stream: int, seed: int):
    """One uniform in [0, 1) per token: counter = (token, kv_head, layer, stream),
    key from `seed`; u = ((x0 * 2^32 + x1) >> 11) * 2^-53 (53 random bits)."""
    k0, k1 = seed_key(seed)
    token = np.asarray(token, dtype=np.uint64)
    x0, x1, _, _ = philox4x32(token, kv_head, layer, stream, k0, k1)
    top53 = ((x0 << np.uint64(32)) | x1) >> np.uint64(11)
    return top53.astype(np.float64) * 2.0 ** -53
