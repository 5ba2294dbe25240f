"""Pins of the oracle's 2-bit key sketch (oracle/sketch2.py) against its definition:
level grid, rounding to the nearest level, exact reconstruction of on-grid data, the
error bound, the extremes, and a worked example computed by hand."""
import numpy as np

from oracle import sketch2


def test_worked_example_by_hand():
    # one group: min -1, max 2, step 1 -> levels -1, 0, 1, 2; midpoints -0.5, 0.5, 1.5
    row = np.zeros((1, 32), dtype=np.float32)
    vals = [-1.0, 2.0, -0.5, 0.49, 0.5, 1.49, 1.5, 0.0]
    row[0, :8] = vals
    codes, mn, sc = sketch2.quantize_rows(np.tile(row, (1, 4)))
    assert mn[0, 0] == -1.0 and sc[0, 0] == 1.0
    # -1 -> 0; 2 -> 3; -0.5 sits on the first midpoint and goes up; 0.49 -> 1 (level 0);
    # 0.5 -> 2; 1.49 -> 2; 1.5 -> 3; the zeros -> 1
    assert codes[0, :8].tolist() == [0, 3, 1, 1, 2, 2, 3, 1]
    xh = sketch2.dequantize(codes, mn, sc)
    assert xh[0, :8].tolist() == [-1.0, 2.0, 0.0, 0.0, 1.0, 1.0, 2.0, 0.0]


def test_on_grid_data_is_reconstructed_exactly():
    rng = np.random.default_rng(0)
    n = 50
    a = (rng.integers(-256, 256, size=(n, 4)) / 64.0).astype(np.float32)   # dyadic: sums exact
    s = np.float32(0.25) * rng.integers(1, 9, size=(n, 4)).astype(np.float32)
    c = rng.integers(0, 4, size=(n, 4, 32))
    c[:, :, 0] = 0
    c[:, :, 1] = 3                       # both extremes present in every group
    x = (a[:, :, None] + c * s[:, :, None]).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), a[:, :, None].astype(np.float64) + c * s[:, :, None].astype(np.float64))
    codes, mn, sc = sketch2.quantize_rows(x.reshape(n, 128))
    assert np.array_equal(codes.reshape(n, 4, 32), c)
    assert np.array_equal(sketch2.dequantize(codes, mn, sc), x.reshape(n, 128).astype(np.float64))


def test_codes_error_bound_and_extremes():
    rng = np.random.default_rng(1)
    K = rng.normal(size=(400, 128)).astype(np.float32)
    K[7, :32] = 0.5                      # a constant group: step 0
    codes, mn, sc = sketch2.quantize_rows(K)
    assert codes.dtype == np.uint8 and codes.min() >= 0 and codes.max() <= 3
    xh = sketch2.dequantize(codes, mn, sc)
    err = np.abs(xh - K.astype(np.float64)).reshape(400, 4, 32)
    bound = sc.astype(np.float64)[:, :, None] / 2 * (1 + 1e-6) + 1e-7 * np.abs(mn.astype(np.float64))[:, :, None]
    assert np.all(err <= bound)
    assert np.all(xh[7, :32] == 0.5)
    # the minimum of every group is reproduced exactly; the maximum within rounding of sc
    g = K.reshape(400, 4, 32)
    assert np.array_equal(mn, g.min(axis=2))
    top = xh.reshape(400, 4, 32).max(axis=2)
    assert np.all(np.abs(top - g.max(axis=2)) <= 4 * np.spacing(np.abs(g.max(axis=2)) + np.abs(mn)))


def test_sketch_is_the_key_when_levels_suffice():
    # keys that take at most four equally spaced values per group are their own sketch
    K = np.tile(np.array([1.0, -1.0, 0.0, 2.0], dtype=np.float32) * np.float32(0.5), (3, 32))
    K = K.reshape(3, 128).astype(np.float32)
    assert np.array_equal(sketch2.sketch_of(K), K.astype(np.float64))
