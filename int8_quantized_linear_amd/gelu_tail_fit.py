"""Fits the polynomial that the kernels' GELU uses for the standard normal tail.

    python int8_quantized_linear_amd/gelu_tail_fit.py

GELU in its exact form is y * Phi(y), Phi the standard normal distribution function. For
every real y it equals max(y, 0) - |y| * Phi(-|y|), since y Phi(y) = y - y Phi(-y). So the
kernels need only the tail Phi(-z) for z >= 0, which falls from 1/2 to about 6e-16 at z = 8.
Its base-2 logarithm is smooth and bends only mildly over [0, 8], so a polynomial in
u = z / 8 reproduces it closely, and the tail is then one exp2 (v_exp_f32) of that
polynomial: no reciprocal and no range branch.

The fit is a weighted minimax fit (Lawson iterations of weighted least squares on
Chebyshev nodes): the allowed error of the tail at z is the smaller of 1e-5 relative and
1e-7 absolute, so that |y| Phi(-|y|) is accurate to a few 1e-6 relative where it is the
whole result (y < 0), and to about 1e-7 |y| where it is subtracted from y (y > 0).
Coefficients are rounded to fp32; `evaluate` runs the kernels' fp32 order (a multiply
clamped at 1, Horner's fused multiply-adds, exp2, one fused multiply-add), and `report`
measures the result against scipy's log_ndtr and ndtr in fp64. The printed table is the
one in csrc/ql_internal.h.

A second, shorter table serves epilogues whose output is fp16. There the result only has to
land within a small fraction of an fp16 step (at least 4.9e-4 of the value), so the tail is
fitted with one relative error bound everywhere, at degree 7 (about 3.3e-5 relative): four
fewer fused multiply-adds per element.
"""
from __future__ import annotations

import numpy as np

Z = 8.0          # u = min(z / Z, 1)
DEGREE = 11
TAU_REL, TAU_ABS = 1e-5, 1e-7
# the fp16-output table: relative error only (the absolute bound never binds)
DEGREE_F16, TAU_REL_F16, TAU_ABS_F16 = 7, 1e-4, 1.0


def fit(degree: int = DEGREE, npts: int = 20000, tau_rel: float = None, tau_abs: float = None) -> np.ndarray:
    """Coefficients of P (highest power first), rounded to fp32."""
    tau_rel = TAU_REL if tau_rel is None else tau_rel
    tau_abs = TAU_ABS if tau_abs is None else tau_abs
    from scipy.special import log_ndtr
    k = np.arange(npts)
    u = (np.cos(np.pi * (k + 0.5) / npts)[::-1] + 1) / 2
    z = u * Z
    target = log_ndtr(-z) / np.log(2)
    tail = np.exp(log_ndtr(-z))
    tol = np.minimum(tau_abs / tail, tau_rel) / np.log(2)   # allowed error of log2 tail
    V = np.vander(u, degree + 1)
    wl = np.ones_like(u)
    for _ in range(400):
        w = np.sqrt(wl) / tol
        c, *_ = np.linalg.lstsq(V * w[:, None], target * w, rcond=None)
        e = np.abs(V @ c - target) / tol
        wl = wl * e
        wl /= wl.sum()
    return c.astype(np.float32)


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _fma32(a, b, c):
    # the exact product plus c, rounded once (an fp64 sum of fp32 operands is exact here up
    # to the final rounding in all but double-rounding corner cases)
    return _f32(np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64))


def evaluate(y, c) -> np.ndarray:
    """GELU in the kernels' fp32 order."""
    y = _f32(y)
    z = np.abs(y)
    u = np.minimum(_f32(z * np.float32(1.0 / Z)), np.float32(1.0))
    p = np.full_like(u, c[0])
    for ci in c[1:]:
        p = _fma32(p, u, np.full_like(u, ci))
    q = _f32(np.exp2(p.astype(np.float64)))
    return _fma32(-z, q, np.maximum(y, np.float32(0.0)))


def report(c) -> dict:
    from scipy.special import ndtr
    y = np.linspace(-12, 12, 2000001).astype(np.float32)
    ref = y.astype(np.float64) * ndtr(y.astype(np.float64))
    err = np.abs(evaluate(y, c) - ref)
    neg = (y < -1e-6) & (y > -6)
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    ref16 = (h.astype(np.float64) * ndtr(h.astype(np.float64))).astype(np.float16)
    out16 = evaluate(h, c).astype(np.float16)
    return {"max_err_over_abs_y": float((err / np.maximum(np.abs(y), 1e-30)).max()),
            "max_rel_err_y_in_(-6,0)": float((err / np.abs(ref))[neg].max()),
            "fp16_inputs_not_correctly_rounded": int((out16 != ref16).sum()),
            "fp16_inputs": int(len(h))}


def fit_f16() -> np.ndarray:
    """The shorter table of the fp16-output epilogues."""
    return fit(DEGREE_F16, tau_rel=TAU_REL_F16, tau_abs=TAU_ABS_F16)


if __name__ == "__main__":
    for name, c in (("c", fit()), ("c16", fit_f16())):
        print(report(c))
        print("constexpr float %s[%d] = {" % (name, len(c)))
        print("    " + ", ".join("%.9ef" % v for v in c) + "};")
