"""A 2-bit key sketch: quantiser and dequantiser (test infrastructure for the oracle only).

The pages evaluate KVFetch with a "2-bit sketch" besides the perfect one (VerKV summary
page, evaluation, the error-bound guarantee results) but define no quantiser.  The
reading taken here: asymmetric uniform quantisation per token row in groups of 32
dimensions (the per-token grouping KIVI uses for 2-bit caches, a paper on the pages'
related-work list), four levels per group:

    mn = min of the group, mx = max of the group            (float32, exact)
    sc = (mx - mn) / 3                                      (float32 division)
    code_j = #{c in 0, 1, 2 : x_j >= mn + (c + 1/2) sc}     (midpoints in float64)
    x_hat_j = mn + code_j * sc                              (float64)

Every step is a single IEEE operation on float32 or float64 values, so a second
implementation that performs the same operations reaches the same codes bit for bit.
The sketch weights of KVFetch step 1 are then computed from x_hat instead of the keys.
"""
from __future__ import annotations

import numpy as np

GROUP = 32          # dimensions per quantisation group
LEVELS = 4          # 2 bits


def quantize_rows(K: np.ndarray):
    """K: [n][d] key rows (bf16 or float32 values, d a multiple of 32).
    Returns codes [n][d] uint8 in 0..3, mn [n][d/32] float32, sc [n][d/32] float32."""
    x = np.asarray(K, dtype=np.float32)
    n, d = x.shape
    assert d % GROUP == 0
    xg = x.reshape(n, d // GROUP, GROUP)
    mn = xg.min(axis=2)
    mx = xg.max(axis=2)
    sc = (mx - mn) / np.float32(LEVELS - 1)                     # float32 / float32
    assert sc.dtype == np.float32
    x64 = xg.astype(np.float64)
    mn64 = mn.astype(np.float64)[:, :, None]
    sc64 = sc.astype(np.float64)[:, :, None]
    codes = np.zeros(xg.shape, dtype=np.uint8)
    for c in range(LEVELS - 1):
        mid = mn64 + (c + 0.5) * sc64
        codes += (x64 >= mid).astype(np.uint8)
    return codes.reshape(n, d), mn, sc


def dequantize(codes: np.ndarray, mn: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """x_hat [n][d] float64 from the codes and the per-group float32 parameters."""
    n, d = codes.shape
    cg = codes.reshape(n, d // GROUP, GROUP).astype(np.float64)
    xh = mn.astype(np.float64)[:, :, None] + cg * sc.astype(np.float64)[:, :, None]
    return xh.reshape(n, d)


def sketch_of(K: np.ndarray) -> np.ndarray:
    """The dequantised 2-bit sketch of key rows K [n][d] (float64)."""
    return dequantize(*quantize_rows(K))
