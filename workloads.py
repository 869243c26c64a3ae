"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random floating-point tensors. It holds none of the
method's arithmetic (no scale, rounding, clamping or packing): the CPU oracle and
the HIP library each quantize what is drawn here on their own.

Every draw uses ``numpy.random.default_rng(seed)`` (PCG64). Draws happen in a
fixed order: the per-column spread vector, W, X, the outlier columns, the bias.
Normal draws are fp32; fp16 tensors are the fp32 draw rounded to nearest-even by
``astype(np.float16)``.

Layouts follow the statement of the problem on hotelren.com "量化算法的本质"
(section on the quantized matrix multiplication's parameters): X is [M, K]
row-major, W is [K, N] stored column-major, which in memory is an [N, K]
row-major array (``w_nk`` below, K contiguous). Bias is [N].

No public benchmark or dataset is used anywhere: the pages measure on
Llama-2-7B / LLaMA-7B layers and calibrate on WikiText-103; these recipes stand
in for them with Llama-7B-shaped synthetic tensors.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "w8a8" | "w8a16" | "w8a16_block" | "w4a16"
    M: int
    K: int
    N: int
    x_dtype: str         # "f32" | "f16"
    y_dtype: str         # "f32" | "f16"
    seed: int
    sigma_lo: float      # per-column spread: exp(U(ln lo, ln hi))
    sigma_hi: float
    sigma_base: float    # W[n, k] = base * spread_n * N(0, 1)
    n_outliers: int      # outlier columns of X, multiplied after drawing
    outlier_gain: float
    bias_std: Optional[float]
    group: int = 0       # block (w8a16_block) or group (w4a16) size along K


# The five workloads. The seed is the workload's number (1..5).
W8A8_SMALL = Workload("w8a8_m16_k256_n256", "w8a8", 16, 256, 256, "f32", "f32", 1,
                      0.005, 0.5, 1.0, 2, 20.0, 0.1)
W8A16_DECODE = Workload("w8a16_m1_k4096_n4096", "w8a16", 1, 4096, 4096, "f16", "f16", 2,
                        0.2, 5.0, 0.02, 0, 1.0, None)
W8A8_PREFILL = Workload("w8a8_m2048_k4096_n11008", "w8a8", 2048, 4096, 11008, "f16", "f16", 3,
                        0.2, 5.0, 0.02, 4, 30.0, 0.1)
W8A16_BLOCK = Workload("w8a16blk64_m8_k4096_n4096", "w8a16_block", 8, 4096, 4096, "f16", "f16", 4,
                       0.2, 5.0, 0.02, 0, 1.0, None, group=64)
W4A16_GROUP = Workload("w4a16g128_m32_k4096_n14336", "w4a16", 32, 4096, 14336, "f16", "f16", 5,
                       0.2, 5.0, 0.02, 0, 1.0, None, group=128)

ALL = (W8A8_SMALL, W8A16_DECODE, W8A8_PREFILL, W8A16_BLOCK, W4A16_GROUP)


def with_shape(w: Workload, M: int, K: int, N: int, seed: Optional[int] = None) -> Workload:
    """The same distributions at another shape (parity cases: ragged, tiny, several tiles)."""
    from dataclasses import replace
    return replace(w, M=M, K=K, N=N, seed=w.seed if seed is None else seed,
                   n_outliers=min(w.n_outliers, K))


@dataclass
class Inputs:
    x: np.ndarray                 # [M, K] float32 or float16
    w_nk: np.ndarray              # [N, K] float32 (W [K, N] column-major)
    bias: Optional[np.ndarray]    # [N] float32 or None
    outlier_cols: np.ndarray      # indices into K


def draw(w: Workload, x_rows: Optional[slice] = None) -> Inputs:
    """Draw one workload's float inputs. ``x_rows`` optionally keeps a row slice of X
    (the full X is still drawn so that the stream of random numbers is unchanged)."""
    rng = np.random.default_rng(w.seed)
    spread = np.exp(rng.uniform(np.log(w.sigma_lo), np.log(w.sigma_hi), size=w.N)).astype(np.float32)
    z = rng.standard_normal((w.N, w.K), dtype=np.float32)
    w_nk = (np.float32(w.sigma_base) * spread[:, None]) * z
    del z
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    if w.n_outliers:
        cols = rng.choice(w.K, w.n_outliers, replace=False)
        x[:, cols] *= np.float32(w.outlier_gain)
    else:
        cols = np.zeros(0, dtype=np.int64)
    bias = None
    if w.bias_std is not None:
        bias = (np.float32(w.bias_std) * rng.standard_normal(w.N, dtype=np.float32)).astype(np.float32)
    if w.x_dtype == "f16":
        x = x.astype(np.float16)
    if x_rows is not None:
        x = np.ascontiguousarray(x[x_rows])
    return Inputs(x=x, w_nk=np.ascontiguousarray(w_nk, dtype=np.float32), bias=bias,
                  outlier_cols=np.sort(cols))


def draw_x_only(w: Workload, seed: int) -> np.ndarray:
    """An extra activation batch of the workload's law (for parity seeds beyond the default)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    if w.n_outliers:
        cols = rng.choice(w.K, w.n_outliers, replace=False)
        x[:, cols] *= np.float32(w.outlier_gain)
    return x.astype(np.float16) if w.x_dtype == "f16" else x
