"""The seeded input recipes: shapes, dtypes, determinism and the stated laws."""
import numpy as np

import workloads


def test_shapes_and_dtypes():
    w = workloads.W8A8_SMALL
    inp = workloads.draw(w)
    assert inp.x.shape == (16, 256) and inp.x.dtype == np.float32
    assert inp.w_nk.shape == (256, 256) and inp.w_nk.dtype == np.float32
    assert inp.bias.shape == (256,) and inp.bias.dtype == np.float32
    assert inp.outlier_cols.size == 2
    small = workloads.with_shape(workloads.W8A8_PREFILL, 40, 256, 300)
    inp = workloads.draw(small)
    assert inp.x.dtype == np.float16 and inp.x.shape == (40, 256)
    assert inp.outlier_cols.size == 4


def test_deterministic_and_seed_dependent():
    a = workloads.draw(workloads.with_shape(workloads.W8A16_DECODE, 1, 512, 64))
    b = workloads.draw(workloads.with_shape(workloads.W8A16_DECODE, 1, 512, 64))
    c = workloads.draw(workloads.with_shape(workloads.W8A16_DECODE, 1, 512, 64, seed=102))
    assert np.array_equal(a.w_nk, b.w_nk) and np.array_equal(a.x, b.x)
    assert not np.array_equal(a.w_nk, c.w_nk)


def test_laws():
    inp = workloads.draw(workloads.with_shape(workloads.W8A8_SMALL, 64, 2048, 256))
    sd = inp.w_nk.std(axis=1)
    assert sd.min() > 0.004 and sd.max() < 0.6
    assert sd.max() / sd.min() > 20          # log-uniform over two decades
    x = inp.x.astype(np.float64)
    cols = inp.outlier_cols
    rest = np.setdiff1d(np.arange(x.shape[1]), cols)
    assert abs(x[:, rest].std() - 1.0) < 0.02
    assert x[:, cols].std() > 10.0           # the x20 outlier columns
    assert abs(inp.bias.std() - 0.1) < 0.03


def test_row_slice_keeps_stream():
    w = workloads.with_shape(workloads.W8A8_PREFILL, 64, 256, 128)
    full = workloads.draw(w)
    part = workloads.draw(w, x_rows=slice(10, 20))
    assert np.array_equal(full.x[10:20], part.x)
    assert np.array_equal(full.w_nk, part.w_nk)
