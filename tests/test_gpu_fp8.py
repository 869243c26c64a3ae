"""GPU parity of the fp8 (OCP E4M3) path: quantizer codes and scales bit-exact against the
oracle; the layer exact where every partial sum is representable, and within a bound
derived from the matrix cores' fp8 arithmetic otherwise.

The fp8 matrix-core step (v_mfma_f32_32x32x64_f8f6f4 on gfx950) does not round like a
chain of fp32 additions. Measured through this library (test_matrix_core_groups pins it):
the 64 products of one step are summed in groups of 8 consecutive k; in each group the
products are aligned to the group's largest exponent sum E = max(e_x + e_w) (unbiased
exponents of the two codes, -6 for subnormals) and each is truncated toward zero to a
multiple of 2^(E - 13); the exact group sum then enters the fp32 accumulator. So
    |y - y64| <= x_scale w_scale sum_g 8 * 2^(E_g - 13)            (truncation)
               + (K/8 + 8) * 2^-24 * (mag + |bias|)                (fp32 sums, epilogue)
with mag = x_scale w_scale sum_k |products| from the oracle; times max |act'| = 1.13
after an activation, plus the activation's own error (the GELU evaluations pinned in
test_gelu_tail: within 6e-6 relative for y in (-6, 0), 3.3e-5 with the shorter tail of fp16
outputs); fp16 outputs add one fp16 step.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, Guarded, dev, f16_ulp, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    import int8_quantized_linear_amd as ql
    return ql


def _codes(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.uint8))


def _check_rows(ql, x: np.ndarray):
    q_ref, s_ref = oracle.quant_rows_e4m3(x)
    xq, xs = ql.quantize_per_row_e4m3(dev(x))
    assert xq.dtype == torch.float8_e4m3fn
    assert np.array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))
    got = _codes(xq)
    bad = got != q_ref
    assert not bad.any(), "%d codes differ; first at %s: %s vs %s (x=%s)" % (
        bad.sum(), np.argwhere(bad)[0], got[bad][:4], q_ref[bad][:4], x[bad][:4])


def test_rows_small(ql):
    _check_rows(ql, workloads.draw(workloads.W8A8_SMALL).x)


def test_rows_prefill_full(ql):
    _check_rows(ql, workloads.draw(workloads.W8A8_PREFILL, x_rows=slice(0, 2048)).x)


@pytest.mark.parametrize("M,K,dtype", [(1, 16, np.float16), (37, 4096, np.float16),
                                       (5, 8256, np.float16), (3, 4112, np.float32),
                                       (64, 48, np.float32), (130, 1024, np.float16), (4, 11008, np.float16), (2, 14336, np.float16), (3, 16400, np.float16), (2, 8208, np.float32)])
def test_rows_shapes(ql, M, K, dtype):
    """Ragged M, the shortest K, and rows too long to keep in registers; row magnitudes
    spread over 2^-8..2^8 so that codes reach E4M3's subnormals."""
    rng = np.random.default_rng(M * 11 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, 1)))).astype(dtype)
    _check_rows(ql, x)


def test_rows_special(ql):
    """Rows whose quotients fall exactly on E4M3 values, on midpoints between neighbours
    (normal and subnormal, both tie directions), on tiny values that round to a signed
    zero, and an all-zero row. With absmax 448 the scale is exactly 1, so x / s = x."""
    K = 64
    rows = []
    v = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], np.float64)   # +0 .. 448
    mids = (v[:-1] + v[1:]) / 2
    r = np.zeros(K, np.float32)
    r[0] = 448.0
    r[1:33] = mids[:32]                     # subnormal and small normal midpoints
    r[33:64] = -mids[64:95]                 # negative normal midpoints
    rows.append(r)
    r = np.zeros(K, np.float32)
    r[0] = -448.0
    r[1:33] = mids[94:126]                  # the largest midpoints (up to 432 .. 448)
    r[33:40] = [-2.0 ** -11, 2.0 ** -11, -1e-6, 1e-6, -0.0, 2.0 ** -10, -2.0 ** -10]
    r[40:64] = v[100:124]                   # exact values
    rows.append(r)
    rows.append(np.zeros(K, np.float32))
    r = np.full(K, -0.0, np.float32)
    r[5] = 3.0
    rows.append(r)
    x = np.stack(rows)
    _check_rows(ql, x)
    _check_rows(ql, x.astype(np.float16))


def test_weight_quantizer(ql):
    inp = workloads.draw(workloads.W8A8_SMALL)
    q_ref, s_ref = oracle.quant_rows_e4m3(inp.w_nk)
    wq, ws = ql.quantize_weight_per_channel_e4m3(dev(inp.w_nk))
    assert np.array_equal(_codes(wq), q_ref)
    assert np.array_equal(host(ws).view(np.uint32), s_ref.view(np.uint32))


def _half_integer_codes(rng, shape) -> np.ndarray:
    """E4M3 codes of j / 2, |j| <= 15: products are multiples of 1/4 below 57, so every
    partial sum over K <= 2^14 is exact in fp32 whatever the order."""
    table = oracle.e4m3_encode((np.arange(-15, 16) / 2).astype(np.float32))
    return table[rng.integers(0, 31, shape)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (16, 256, 256), (300, 520, 384), (257, 129, 192),
                                   (128, 300, 128), (2000, 8300, 256), (64, 256, 4096), (16, 11008, 1024),
                                   (24, 10240, 192), (200, 3001, 576), (1, 4096, 4096), (8, 1000, 1344),
                                   (40, 2000, 704), (20, 4096, 1472), (1000, 4096, 192), (300, 7000, 320),
                                   (600, 9001, 192), (1025, 4100, 192),    # 128 x 192 tiles
                                   (1000, 9001, 192), (768, 11008, 128)])  # 256 x 192 tiles
def test_exact_sums(ql, M, N, K):
    """With unit scales, no bias and fp32 output, y is the exact sum of products: any
    dropped, repeated or misplaced product shows. Covers several tiles, ragged M and N,
    the 64 x 64 kernel (with a half-deep last stage), the mixed big/half tile plan, a long K,
    the tile kernel on 128 x 128 tiles (M = 1000, N = 4096; ragged with a half-deep last stage at
    300 x 7000 x 320), the few-row kernel's four-wave shape (more than 2 x CUs workgroups of 16
    columns), and its eight-wave ring over pairs of steps (2 pairs in flight up to 8 rows, 1 beyond), with odd
    step counts per wave and odd first steps (K = 1344: 21 steps over 8 waves; K = 704, 1472)."""
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a = _half_integer_codes(rng, (M, K))
    b = _half_integer_codes(rng, (N, K))
    ones_m = np.ones(M, np.float32)
    ones_n = np.ones(N, np.float32)
    g = Guarded((M, N), torch.float32)
    ql.gemm_e4m3_per_channel(dev(a), dev(ones_m), dev(b), dev(ones_n), None, "none",
                             torch.float32, y=g.view)
    g.check()
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 61), np.arange(M - 5, M)]))
    y64, _ = oracle.gemm_e4m3_f64(a[rows], ones_m[rows], b, ones_n)
    assert np.array_equal(host(g.view)[rows].astype(np.float64), y64)


def _exp(codes: np.ndarray) -> np.ndarray:
    """Unbiased exponent of each E4M3 code's significand (-6 for zero and subnormals)."""
    e = (codes.astype(np.int16) >> 3) & 15
    return np.where(e == 0, -6, e - 7).astype(np.int16)


def _trunc_bound(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """sum over groups of 8 consecutive k of 8 * 2^(E_g - 13), E_g the group's largest
    exponent sum, for every (row of xq, row of wq): the matrix cores' truncation bound in
    units of code products."""
    ex, ew = _exp(xq), _exp(wq)
    K = ex.shape[1]
    out = np.zeros((ex.shape[0], ew.shape[0]))
    for g in range(0, K, 8):
        e = (ex[:, None, g:g + 8] + ew[None, :, g:g + 8]).max(-1)
        out += np.exp2(e - 10.0)
    return out


def _layer_tol(y64, mag, trunc, K, code, out):
    ref = oracle.activation_f64(y64, code)
    act_err = 3.3e-5 if out == torch.float16 else 6e-6
    tol = (1.13 if code else 1.0) * (trunc + (K / 8 + 8) * 2.0 ** -24 * mag) + act_err * np.abs(ref)
    if out == torch.float16:
        tol = tol + f16_ulp(ref)
    return ref, tol


@pytest.mark.parametrize("M,N,K,out,act", [(16, 256, 256, torch.float32, "none"),
                                           (300, 520, 384, torch.float16, "none"),
                                           (257, 129, 192, torch.float32, "gelu"),
                                           (100, 1000, 384, torch.float16, "silu"),
                                           (100, 1000, 384, torch.float16, "gelu"),
                                           (2048, 11008, 4096, torch.float16, "none"),
                                           (600, 9001, 256, torch.float32, "gelu"),    # 128 x 192 tiles
                                           (1000, 9001, 256, torch.float16, "none")])  # 256 x 192 tiles
def test_layer(ql, M, N, K, out, act):
    """The whole fp8 layer (both quantizers on the GPU) against the oracle's fp8 layer in
    fp64 on the oracle's own codes. Quantization is per row of X and per column of W, so
    the oracle quantizes only the sampled rows and columns (all of them up to 512; at the
    prefill shape rows from every 128-row band and columns from every 64-column panel);
    the GPU's codes are compared bit-exactly there."""
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N)
    inp = workloads.draw(w)
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    cols = np.arange(N) if N <= 1024 else np.unique(np.concatenate([np.arange(0, N, 41), [N - 1]]))
    wq_r, ws_r = oracle.quant_rows_e4m3(inp.w_nk[cols])
    xq_r, xs_r = oracle.quant_rows_e4m3(inp.x[rows])
    wq, ws = ql.quantize_weight_per_channel_e4m3(dev(inp.w_nk))
    xq, xs = ql.quantize_per_row_e4m3(dev(inp.x))
    assert np.array_equal(_codes(wq)[cols], wq_r)
    assert np.array_equal(host(ws)[cols].view(np.uint32), ws_r.view(np.uint32))
    assert np.array_equal(_codes(xq)[rows], xq_r)
    assert np.array_equal(host(xs)[rows].view(np.uint32), xs_r.view(np.uint32))
    g = Guarded((M, N), out)
    ql.gemm_e4m3_per_channel(xq, xs, wq, ws, dev(inp.bias), act, out, y=g.view)
    g.check()
    y64, mag = oracle.gemm_e4m3_f64(xq_r, xs_r, wq_r, ws_r, inp.bias[cols])
    mag = mag + np.abs(inp.bias[cols].astype(np.float64))[None, :]
    trunc = (xs_r.astype(np.float64)[:, None] * ws_r.astype(np.float64)[None, :]) * _trunc_bound(xq_r, wq_r)
    ref, tol = _layer_tol(y64, mag, trunc, K, {"none": 0, "gelu": 1, "silu": 2}[act], out)
    y = host(g.view)[np.ix_(rows, cols)].astype(np.float64)
    err = np.abs(y - ref)
    assert np.all(err <= tol), "max err/tol %.3g" % float((err / tol).max())


@pytest.mark.parametrize("rows", ["few", "mid", "tiles"])
def test_matrix_core_groups(ql, rows):
    """The premises of the bound above, on all three kernels: up to 128 rows the few-row kernel
    (16x16x128 fp8 steps); 160 rows against 160 columns the 64 x 64 kernel, and against 33024
    columns (more tiles than the 64 x 64 kernel takes) the tile kernel, both on 32x32x64 steps.
    The cases are padded with zero rows and columns. One output each (unit scales, K = 64,
    fp32 out): a
    product of 4 beside 2^16 (2^-14 of it) vanishes when both lie in one group of 8
    consecutive k and survives in another group; a product of +-28 beside 2^16 keeps
    +-24 (truncation toward zero to multiples of 2^(16 - 13)); 2^16 + 2^-7 across groups
    is exact (fp32 accumulation of group sums); subnormal codes multiply exactly."""
    enc = lambda v: int(oracle.e4m3_encode(np.float32(v)))
    cases = []
    for j in range(1, 64):
        cases.append(({0: 256.0, j: 1.0}, {0: 256.0, j: 4.0}, 65536.0 if j < 8 else 65540.0))
    for base in (8, 27, 56):
        cases.append(({base: 256.0, base ^ 1: 1.0}, {base: 256.0, base ^ 1: 4.0}, 65536.0))
    cases.append(({0: 256.0, 1: 1.75}, {0: 256.0, 1: 16.0}, 65560.0))
    cases.append(({0: 256.0, 1: -1.75}, {0: 256.0, 1: 16.0}, 65512.0))
    cases.append(({0: 256.0, 1: 1.5}, {0: 256.0, 1: 16.0}, 65560.0))
    cases.append(({0: 256.0, 63: 0.125}, {0: 256.0, 63: 0.0625}, 65536.0 + 2.0 ** -7))
    cases.append(({3: 2.0 ** -9}, {3: 2.0 ** -9}, 2.0 ** -18))
    cases.append(({9: 3 * 2.0 ** -9}, {9: 5 * 2.0 ** -9}, 15 * 2.0 ** -18))
    R = len(cases)
    M = (R + 31) // 32 * 32 if rows == "few" else 160
    N = 33024 if rows == "tiles" else M
    assert (M <= 128) == (rows == "few")
    A = np.zeros((M, 64), np.uint8)
    B = np.zeros((N, 64), np.uint8)
    for r, (a, b, _) in enumerate(cases):
        for k, v in a.items():
            A[r, k] = enc(v)
        for k, v in b.items():
            B[r, k] = enc(v)
    y = host(ql.gemm_e4m3_per_channel(dev(A), dev(np.ones(M, np.float32)), dev(B), dev(np.ones(N, np.float32)),
                                      out_dtype=torch.float32))
    got = np.array([y[r, r] for r in range(R)], np.float64)
    want = np.array([c[2] for c in cases])
    assert np.array_equal(got, want), [(r, got[r], want[r]) for r in range(R) if got[r] != want[r]][:6]


def test_raw_byte_codes_match_fp8_tensors(ql):
    """uint8 code tensors and float8_e4m3fn tensors are the same bytes to the library."""
    rng = np.random.default_rng(5)
    a = _half_integer_codes(rng, (40, 128))
    b = _half_integer_codes(rng, (72, 128))
    xs = np.full(40, 0.5, np.float32)
    ws = np.full(72, 0.25, np.float32)
    y1 = ql.gemm_e4m3_per_channel(dev(a), dev(xs), dev(b), dev(ws), out_dtype=torch.float32)
    y2 = ql.gemm_e4m3_per_channel(dev(a).view(torch.float8_e4m3fn), dev(xs),
                                  dev(b).view(torch.float8_e4m3fn), dev(ws), out_dtype=torch.float32)
    assert torch.equal(y1, y2)


def test_empty(ql):
    xq = torch.empty((0, 64), dtype=torch.float8_e4m3fn, device=DEV)
    wq = torch.zeros((8, 64), dtype=torch.float8_e4m3fn, device=DEV)
    y = ql.gemm_e4m3_per_channel(xq, torch.empty(0, device=DEV), wq, torch.ones(8, device=DEV))
    assert y.shape == (0, 8)
