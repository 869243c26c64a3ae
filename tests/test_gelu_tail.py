"""The GELU that the kernels' epilogues evaluate (csrc/ql_internal.h, normal_tail and
activation), run here in the same fp32 order from the coefficient table in the header,
against y * Phi(y) in fp64 (scipy). Pins the accuracy the header states: within 1e-7 |y|
for every y, within 6e-6 relative for y in (-6, 0), and within one fp16 step of the
correctly rounded fp16 value for every finite fp16 input. The kernels' GELU itself is
checked on the GPU against the oracle's fp64 activation (test_gpu_w8a8, test_gpu_wonly)."""
import os
import re

import numpy as np
import pytest

scipy = pytest.importorskip("scipy")

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_fit():
    # by path: importing the package would load libql.so, which this test does not need
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "gelu_tail_fit", os.path.join(HERE, "..", "int8_quantized_linear_amd", "gelu_tail_fit.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


fit = _load_fit()
HEADER = os.path.join(HERE, "..", "int8_quantized_linear_amd", "csrc", "ql_internal.h")


def header_table():
    src = open(HEADER).read()
    body = re.search(r"normal_tail\(float z\) \{\s*constexpr float c\[12\] = \{([^}]*)\}", src).group(1)
    return np.array([float(v.rstrip("f")) for v in body.replace("\n", " ").split(",")], dtype=np.float32)


def test_table_accuracy():
    r = fit.report(header_table())
    assert r["max_err_over_abs_y"] <= 1e-7
    assert r["max_rel_err_y_in_(-6,0)"] <= 6e-6
    assert r["fp16_inputs_not_correctly_rounded"] <= 5


def test_fp16_within_one_step():
    from scipy.special import ndtr
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    ref = (h.astype(np.float64) * ndtr(h.astype(np.float64))).astype(np.float16)
    out = fit.evaluate(h.astype(np.float32), header_table()).astype(np.float16)
    with np.errstate(over="ignore"):
        step = np.spacing(np.abs(ref)).astype(np.float64)
    assert np.all(np.abs(out.astype(np.float64) - ref.astype(np.float64)) <= step)


def test_special_values():
    c = header_table()
    y = np.array([0.0, -0.0, 1e-30, -1e-30, 8.0, -8.0, 30.0, -30.0, 1e4, -1e4], dtype=np.float32)
    g = fit.evaluate(y, c)
    assert g[0] == 0.0 and g[1] == 0.0
    assert g[6] == np.float32(30.0) and g[8] == np.float32(1e4)
    # far negative: the tail stays at Phi(-8) ~ 6.2e-16, so |GELU| <= 6.3e-16 |y|
    assert abs(g[7]) <= 6.3e-16 * 30 and abs(g[9]) <= 6.3e-16 * 1e4
    assert np.float16(g[9]) == 0.0


def test_fit_reproduces_table():
    """The committed table is what the fitting script produces (to the last few fp32 bits:
    least squares may round differently on another BLAS)."""
    assert np.allclose(fit.fit(), header_table(), rtol=1e-5, atol=0)
