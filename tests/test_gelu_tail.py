"""The GELU that the kernels' epilogues evaluate (csrc/ql_internal.h, normal_tail and
activation), run here in the same fp32 order from the coefficient table in the header,
against y * Phi(y) in fp64 (scipy). Pins the accuracy the header states: within 1e-7 |y|
for every y, within 6e-6 relative for y in (-6, 0), and within one fp16 step of the
correctly rounded fp16 value for every finite fp16 input. The shorter table of the
fp16-output epilogues (normal_tail_f16out) is pinned to what fp16 outputs need: within one
fp16 step of the correctly rounded value for every finite fp16 input, within 3.3e-5 relative
for y in (-6, 0) and 1.6e-5 |y| everywhere. The kernels' GELU itself is checked on the GPU
against the oracle's fp64 activation (test_gpu_w8a8, test_gpu_wonly)."""
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


def header_table(name="normal_tail", array="c", n=12):
    src = open(HEADER).read()
    body = re.search(name + r"\(float z\) \{\s*constexpr float " + array + r"\[" + str(n) + r"\] = \{([^}]*)\}",
                     src).group(1)
    return np.array([float(v.rstrip("f")) for v in body.replace("\n", " ").split(",")], dtype=np.float32)


def header_table_f16():
    return header_table("normal_tail_f16out", "c16", 8)


def test_table_accuracy():
    r = fit.report(header_table())
    assert r["max_err_over_abs_y"] <= 1e-7
    assert r["max_rel_err_y_in_(-6,0)"] <= 6e-6
    assert r["fp16_inputs_not_correctly_rounded"] <= 5


def test_table_f16_accuracy():
    r = fit.report(header_table_f16())
    assert r["max_err_over_abs_y"] <= 1.6e-5
    assert r["max_rel_err_y_in_(-6,0)"] <= 3.3e-5


@pytest.mark.parametrize("table", [header_table, header_table_f16])
def test_fp16_within_one_step(table):
    from scipy.special import ndtr
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    ref = (h.astype(np.float64) * ndtr(h.astype(np.float64))).astype(np.float16)
    out = fit.evaluate(h.astype(np.float32), table()).astype(np.float16)
    with np.errstate(over="ignore"):
        step = np.spacing(np.abs(ref)).astype(np.float64)
    assert np.all(np.abs(out.astype(np.float64) - ref.astype(np.float64)) <= step)


def test_fp16_margin_of_short_table():
    """The fp16 pre-activation values that a kernel rounds from fp32 are not exactly the fp16
    grid: over fp32 inputs spread through [-12, 12], the short table's result stays within a
    tenth of an fp16 step of y Phi(y) (so the output lands within one step after rounding)."""
    from scipy.special import ndtr
    y = np.linspace(-12, 12, 2000001).astype(np.float32)
    ref = y.astype(np.float64) * ndtr(y.astype(np.float64))
    out = fit.evaluate(y, header_table_f16()).astype(np.float64)
    with np.errstate(over="ignore"):
        step = np.spacing(np.abs(ref.astype(np.float16))).astype(np.float64)
    assert np.all(np.abs(out - ref) <= 0.1 * step)


@pytest.mark.parametrize("table", [header_table, header_table_f16])
def test_special_values(table):
    c = table()
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
    assert np.allclose(fit.fit_f16(), header_table_f16(), rtol=1e-5, atol=0)
