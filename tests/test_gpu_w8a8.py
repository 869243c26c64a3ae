"""GPU parity of the W8A8 path: int32 accumulators bit-exact, outputs within tolerance.

Tolerances (derived from the arithmetic, since the accumulators are exact):
  fp32 output: |y - y64| <= 1e-5 * (|acc * xs * ws| + |bias|); the only error is the
               few fp32 roundings of the epilogue (about 4 * 2^-24 of that magnitude).
  fp16 output: |y - fp16(y32)| <= one fp16 ulp at the oracle's value, where y32 is the
               oracle's fp32 epilogue; fp32 reordering can move a value across an fp16
               rounding boundary but by no more than one step.
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


def _rand_codes(rng, shape, lo=-127):
    return rng.integers(lo, 128, shape, dtype=np.int8)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (16, 256, 256), (300, 520, 384), (257, 129, 192),
                                   (512, 768, 1024), (33, 1000, 192), (256, 256, 64),
                                   (100, 1000, 384), (128, 300, 128), (64, 256, 640), (127, 513, 256)])
def test_int32_bit_exact(ql, M, N, K):
    """Several tiles in M and N, ragged tails, K with a half k-tile tail, codes including -128,
    with 1, 2, 3 and 5 128-deep stages: small M on the few-row kernel, the others on the 64 x 64
    kernel (the 256 x 256 / 128 x 256 tile kernel's plans are covered below)."""
    rng = np.random.default_rng(M * 1000 + N + K)
    a = _rand_codes(rng, (M, K), -128)
    b = _rand_codes(rng, (N, K), -128)
    acc = ql.gemm_w8a8_int32(dev(a), dev(b))
    assert np.array_equal(host(acc), oracle.gemm_i32(a, b))


@pytest.mark.parametrize("M,N,K", [(2000, 8300, 64), (2048, 11008, 192), (2048, 11008, 384),
                                   (2000, 8300, 256), (4096, 8400, 128), (8192, 2100, 64),
                                   (768, 11008, 256), (1000, 9001, 192), (1280, 8192, 320),
                                   (768, 11008, 64), (2048, 11008, 64)])   # one half-deep stage
def test_int32_mixed_tile_plan(ql, M, N, K):
    """Shapes with more 256 x 256 tiles than CUs, where the last N panels run as 128-row
    tiles in the same launch, each after a big tile in the same workgroup or, with one round
    of big tiles, before it on half of the workgroups (the staggered order; ragged M and N
    in the first case; two rounds of big tiles before the half tiles in the fifth; a ragged
    half-tile panel in the last); and shapes whose 256 x 256 tiles would make one partial
    round, run as 256 x 192 tiles (ragged M and N, a half-deep last stage); rows sampled from
    every 128-row band are checked bit-exactly."""
    rng = np.random.default_rng(M + N + K)
    a = _rand_codes(rng, (M, K), -128)
    b = _rand_codes(rng, (N, K), -128)
    acc = host(ql.gemm_w8a8_int32(dev(a), dev(b)))
    rows = np.unique(np.concatenate([np.arange(0, M, 61), np.arange(M - 5, M)]))
    assert np.array_equal(acc[rows], oracle.gemm_i32(a[rows], b))


def test_int32_extremes(ql):
    """The largest K the boundary accepts with the most negative products."""
    K = 131008
    a = np.full((20, K), 127, np.int8)
    b = np.full((17, K), -128, np.int8)
    acc = host(ql.gemm_w8a8_int32(dev(a), dev(b)))
    assert np.all(acc == np.int64(127) * -128 * K)


@pytest.mark.parametrize("M", [1, 9, 40])
def test_int32_largest_n(ql, M):
    """N = 2^23, the largest the boundary accepts: the few-row kernel at one row, the tile
    kernel's small tiles at 9 and 40 rows (32,768 workgroups), where a band of 32 output rows
    of int32 spans 2^30 bytes less the last piece. Columns sampled across the whole width and
    at its end, bit for bit."""
    N, K = 1 << 23, 64
    rng = np.random.default_rng(M + 23)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    g = Guarded((M, N), torch.int32)
    ql.gemm_w8a8_int32(dev(a), dev(b), acc=g.view)
    g.check()
    cols = np.unique(np.concatenate([np.arange(0, N, 4093), np.arange(N - 300, N)]))
    assert np.array_equal(host(g.view)[:, cols], oracle.gemm_i32(a, b[cols]))


def _layer(ql, w: workloads.Workload, rows=None):
    inp = workloads.draw(w, x_rows=rows)
    wq_ref, ws_ref = oracle.quant_weight_per_channel(inp.w_nk)
    xq_ref, xs_ref = oracle.quant_rows_i8(inp.x)
    wq, ws = ql.quantize_weight_per_channel(dev(inp.w_nk))
    xq, xs = ql.quantize_per_row_int8(dev(inp.x))
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(ws), ws_ref)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(xs), xs_ref)
    return inp, (xq, xs, wq, ws), (xq_ref, xs_ref, wq_ref, ws_ref)


def test_small_layer_fp32(ql):
    """M=16 K=256 N=256 with fp32 output: the whole layer against the oracle."""
    inp, (xq, xs, wq, ws), (xq_r, xs_r, wq_r, ws_r) = _layer(ql, workloads.W8A8_SMALL)
    acc_ref = oracle.gemm_i32(xq_r, wq_r)
    assert np.array_equal(host(ql.gemm_w8a8_int32(xq, wq)), acc_ref)
    y32, y64 = oracle.epilogue_w8a8(acc_ref, xs_r, ws_r, inp.bias)
    y = host(ql.gemm_w8a8_per_channel(xq, xs, wq, ws, dev(inp.bias), torch.float32)).astype(np.float64)
    mag = np.abs(acc_ref.astype(np.float64) * xs_r[:, None] * ws_r[None, :]) + np.abs(inp.bias)[None, :]
    assert np.all(np.abs(y - y64) <= 1e-5 * mag)
    # and the one-call layer
    y2 = host(ql.linear_w8a8(dev(inp.x), wq, ws, dev(inp.bias))).astype(np.float64)
    assert np.array_equal(y2, y)


def test_prefill_full_size(ql):
    """M=2048 K=4096 N=11008 in the benchmark's launch configuration: quantized tensors,
    all 22.5 M int32 accumulators bit for bit, and every fp16 output within one fp16 step of
    the oracle's fp32 epilogue (the oracle's whole GEMM takes a few seconds on the host)."""
    inp, (xq, xs, wq, ws), (xq_r, xs_r, wq_r, ws_r) = _layer(ql, workloads.W8A8_PREFILL)
    y = ql.gemm_w8a8_per_channel(xq, xs, wq, ws, dev(inp.bias), torch.float16)
    acc = ql.gemm_w8a8_int32(xq, wq)
    acc_ref = oracle.gemm_i32(xq_r, wq_r)
    assert np.array_equal(host(acc), acc_ref)
    y32, y64 = oracle.epilogue_w8a8(acc_ref, xs_r, ws_r, inp.bias)
    yg = host(y)
    assert np.all(np.isfinite(yg))
    ref16 = y32.astype(np.float16).astype(np.float64)
    assert np.all(np.abs(yg.astype(np.float64) - ref16) <= f16_ulp(ref16))
    same = np.mean(yg == y32.astype(np.float16))
    assert same > 0.99, same


@pytest.mark.parametrize("M,N,K,with_bias,out", [(300, 520, 384, True, torch.float16),
                                                 (300, 520, 384, False, torch.float16),
                                                 (1, 77, 64, True, torch.float32),
                                                 (513, 300, 640, True, torch.float32),
                                                 (600, 9001, 256, True, torch.float32),    # 128 x 192 tiles,
                                                 (1025, 4100, 192, False, torch.float16),   # scalar stores
                                                 (1000, 9001, 256, True, torch.float32),   # 256 x 192 tiles
                                                 (768, 11008, 256, True, torch.float16)])
def test_ragged_layer(ql, M, N, K, with_bias, out):
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N)
    inp, (xq, xs, wq, ws), (xq_r, xs_r, wq_r, ws_r) = _layer(ql, w)
    bias = inp.bias if with_bias else None
    g = Guarded((M, N), out)
    ql.gemm_w8a8_per_channel(xq, xs, wq, ws, dev(bias) if with_bias else None, out, y=g.view)
    g.check()
    acc_ref = oracle.gemm_i32(xq_r, wq_r)
    y32, y64 = oracle.epilogue_w8a8(acc_ref, xs_r, ws_r, bias)
    y = host(g.view).astype(np.float64)
    if out == torch.float32:
        mag = np.abs(acc_ref.astype(np.float64) * xs_r[:, None] * ws_r[None, :])
        if with_bias:
            mag = mag + np.abs(bias)[None, :]
        assert np.all(np.abs(y - y64) <= 1e-5 * mag)
    else:
        ref16 = y32.astype(np.float16).astype(np.float64)
        assert np.all(np.abs(y - ref16) <= f16_ulp(ref16))


def test_one_hot_rows(ql):
    """X = e_k rows: every output is 127 * wq[k, n] in the accumulators."""
    K, N = 256, 300
    rng = np.random.default_rng(9)
    wq = _rand_codes(rng, (N, K))
    ks = np.array([0, 1, 63, 64, 128, 255])
    a = np.zeros((ks.size, K), np.int8)
    a[np.arange(ks.size), ks] = 127
    acc = host(ql.gemm_w8a8_int32(dev(a), dev(wq)))
    assert np.array_equal(acc, 127 * wq[:, ks].T.astype(np.int32))


ACT = {"gelu": 1, "silu": 2}


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("M,N,K,out", [(16, 256, 256, torch.float32), (300, 520, 384, torch.float16),
                                       (300, 520, 384, torch.float32), (2000, 8300, 64, torch.float16),
                                       (600, 9001, 256, torch.float32),    # 128 x 192 tiles
                                       (1000, 9001, 256, torch.float16),   # 256 x 192 tiles
                                       (16, 4096, 256, torch.float16),     # few-row kernel
                                       (256, 4096, 256, torch.float16),    # mid-size M
                                       (2048, 11008, 4096, torch.float16)])  # the prefill plan
def test_fused_activation(ql, act, M, N, K, out):
    """act(acc * x_scale * w_scale + bias) from the epilogue, against the oracle's fp64
    activation of its fp64 epilogue; half-height-only, mixed and big-tile plans.
    Scales put the pre-activation values at a few units, where both activations bend.
    fp32: |y - act(y64)| <= 1.2e-5 * (|acc xs ws| + |bias|) + 6e-6 |act(y64)| (the
    epilogue's error times |act'| <= 1.13, plus the activation's own fp32 evaluation, which
    test_gelu_tail pins within 6e-6 relative for GELU on y in (-6, 0));
    fp16: within one fp16 step of fp16(act(y64)) (fp16 outputs take the shorter tail, which
    test_gelu_tail pins within a tenth of an fp16 step of y Phi(y))."""
    rng = np.random.default_rng(M + 7 * N + K)
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    xs = (rng.uniform(0.5, 1.5, M) / (127.0 * np.sqrt(K))).astype(np.float32)
    ws = (rng.uniform(0.5, 1.5, N) * 3.0 / 127.0).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    g = Guarded((M, N), out)
    ql.gemm_w8a8_per_channel_act(dev(a), dev(xs), dev(b), dev(ws), dev(bias), act, out, y=g.view)
    g.check()
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 37), [M - 1]]))
    acc_ref = oracle.gemm_i32(a[rows], b)
    _, y64 = oracle.epilogue_w8a8(acc_ref, xs[rows], ws, bias)
    ref = oracle.activation_f64(y64, ACT[act])
    y = host(g.view)[rows].astype(np.float64)
    assert np.all(np.isfinite(y))
    if out == torch.float32:
        mag = np.abs(acc_ref.astype(np.float64) * xs[rows][:, None] * ws[None, :]) + np.abs(bias)[None, :]
        assert np.all(np.abs(y - ref) <= 1.2e-5 * mag + 6e-6 * np.abs(ref))
    else:
        ref16 = ref.astype(np.float16).astype(np.float64)
        assert np.all(np.abs(y - ref16) <= f16_ulp(ref16))
    # the pre-activation values span the bend of both activations
    assert (y64 < -2).mean() > 0.05 and (y64 > 2).mean() > 0.05


def test_fused_activation_none_is_plain(ql):
    """act = none through the activation entry point is the plain epilogue, bit for bit."""
    rng = np.random.default_rng(5)
    M, N, K = 300, 520, 384
    a, b = dev(_rand_codes(rng, (M, K))), dev(_rand_codes(rng, (N, K)))
    xs, ws = dev(rng.uniform(1e-5, 1e-4, M).astype(np.float32)), dev(rng.uniform(1e-3, 1e-2, N).astype(np.float32))
    bias = dev(rng.standard_normal(N).astype(np.float32))
    y0 = host(ql.gemm_w8a8_per_channel(a, xs, b, ws, bias, torch.float16))
    y1 = host(ql.gemm_w8a8_per_channel_act(a, xs, b, ws, bias, "none", torch.float16))
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))


@pytest.mark.parametrize("M,N,K,out,act", [(1, 4096, 4096, torch.float16, "none"), (33, 520, 384, torch.float32, "gelu"), (16, 256, 256, torch.float32, "none"), (300, 520, 384, torch.float16, "none"),
                                           (16, 11008, 512, torch.float16, "silu"),
                                           (257, 129, 192, torch.float32, "gelu"), (2000, 8300, 64, torch.float16, "silu"),
                                           (2048, 11008, 4096, torch.float16, "none"),
                                           (768, 4096, 256, torch.float16, "gelu"),    # 128 x 128 tiles
                                           (600, 9001, 256, torch.float32, "silu"),    # 128 x 192 tiles
                                           (768, 11008, 256, torch.float16, "gelu")])  # 256 x 192 tiles
def test_asymmetric_layer(ql, M, N, K, out, act):
    """Asymmetric activations end to end on the GPU (quantizer bit-exact, column sums exact)
    against the oracle's layer from its definition, sum_k s_x (q_x - z_x) s_w q_w + b.
    The kernel takes acc - z_x colsum with one rounding: fp32 outputs within
    1e-5 (s_x s_w (|acc| + |z_x colsum|) + |b|), times max |act'| = 1.13 when an activation
    follows, plus 6e-6 |act(y64)|; fp16 outputs additionally one fp16 step. Activations
    are ReLU-like on half the rows (non-negative, zero point -128)."""
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N)
    inp = workloads.draw(w)
    x = inp.x.astype(np.float32)
    x[::2] = np.maximum(x[::2], 0)
    x = x.astype(inp.x.dtype)
    wq_r, ws_r = oracle.quant_weight_per_channel(inp.w_nk)
    wq, ws = ql.quantize_weight_per_channel(dev(inp.w_nk))
    cs = ql.weight_column_sums_i8(wq)
    assert np.array_equal(host(cs), oracle.column_sums_i8(wq_r))
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    xq_r, xs_r, xz_r = oracle.quant_rows_i8_asym(x)
    xq, xs, xz = ql.quantize_per_row_int8_asym(dev(x))
    assert np.array_equal(host(xq), xq_r) and np.array_equal(host(xz), xz_r)
    g = Guarded((M, N), out)
    ql.gemm_w8a8_asym(xq, xs, xz, wq, ws, cs, dev(inp.bias), act, out, y=g.view)
    g.check()
    y64 = oracle.w8a8_asym_f64(xq_r[rows], xs_r[rows], xz_r[rows], wq_r, ws_r, inp.bias)
    acc = oracle.gemm_i32(xq_r[rows], wq_r).astype(np.float64)
    colsum = oracle.column_sums_i8(wq_r).astype(np.float64)
    mag = (xs_r[rows].astype(np.float64)[:, None] * ws_r.astype(np.float64)[None, :]
           * (np.abs(acc) + np.abs(xz_r[rows].astype(np.float64)[:, None] * colsum[None, :]))
           + np.abs(inp.bias.astype(np.float64))[None, :])
    code = {"none": 0, "gelu": 1, "silu": 2}[act]
    ref = oracle.activation_f64(y64, code)
    tol = (1.13 if code else 1.0) * 1e-5 * mag + 6e-6 * np.abs(ref)
    y = host(g.view)[rows].astype(np.float64)
    if out == torch.float16:
        tol = tol + f16_ulp(ref)
    assert np.all(np.abs(y - ref) <= tol)


def test_empty(ql):
    xq = torch.empty((0, 64), dtype=torch.int8, device=DEV)
    wq = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    y = ql.gemm_w8a8_per_channel(xq, torch.empty(0, device=DEV), wq, torch.ones(8, device=DEV))
    assert y.shape == (0, 8)


def _requant_case(ql, M, N, K, per_tensor, seed_shift=0):
    """GPU-quantized operands (checked bit for bit), the oracle's fp32 epilogue, and static
    output scales calibrated on another batch of the same law, so that some outputs exceed
    the calibrated maximum and clamp."""
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N)
    inp = workloads.draw(w)
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    wq_r, ws_r = oracle.quant_weight_per_channel(inp.w_nk)
    xq_r, xs_r = oracle.quant_rows_i8(inp.x[rows])
    wq, ws = ql.quantize_weight_per_channel(dev(inp.w_nk))
    xq, xs = ql.quantize_per_row_int8(dev(inp.x))
    assert np.array_equal(host(wq), wq_r) and np.array_equal(host(xq)[rows], xq_r)
    cal = workloads.draw_x_only(w, 101 + seed_shift)[: min(M, 64)]
    cq, cs = oracle.quant_rows_i8(cal)
    y_cal = oracle.epilogue_w8a8(oracle.gemm_i32(cq, wq_r), cs, ws_r, inp.bias)[0]
    s_out = oracle.channel_scales(y_cal) * np.float32(0.9)    # 0.9: some outputs clamp
    if per_tensor:   # the widest channel's scale for all: half of it, so that some clamp
        s_out = np.array([s_out.max() * np.float32(0.5)], np.float32)
    y32, y64 = oracle.epilogue_w8a8(oracle.gemm_i32(xq_r, wq_r), xs_r, ws_r, inp.bias)
    return inp, rows, xq, xs, wq, ws, s_out, y32


@pytest.mark.parametrize("M,N,K,per_tensor", [(1, 4096, 4096, False), (40, 1000, 640, True), (64, 257, 192, False),
                                              (20, 9000, 640, False),
                                              (16, 256, 256, False), (16, 256, 256, True), (300, 520, 384, False),
                                              (257, 129, 192, True), (128, 1000, 128, False),
                                              (2000, 8300, 256, False), (2048, 11008, 4096, True),
                                              (1000, 4096, 256, False),    # 128 x 128 tiles
                                              (600, 9000, 256, False), (1025, 4100, 192, True),    # 128 x 192
                                              (1000, 9001, 192, False), (1280, 8192, 256, True)])  # 256 x 192
def test_requant_bit_exact(ql, M, N, K, per_tensor):
    """int8 output codes bit for bit: the kernel takes ((acc * xs) * ws) + b with separate
    roundings, then the correctly rounded y / s, RNE and the clamp, exactly the oracle's
    fp32 decision. Ragged N (byte stores), half-height, mixed and big tile plans, per-column
    and per-tensor scales, the prefill shape on sampled rows."""
    inp, rows, xq, xs, wq, ws, s_out, y32 = _requant_case(ql, M, N, K, per_tensor)
    g = Guarded((M, N), torch.int8)
    ql.gemm_w8a8_requant(xq, xs, wq, ws, dev(s_out), dev(inp.bias), "none", yq=g.view)
    g.check()
    q_ref = oracle.requant_i8(y32, s_out)
    got = host(g.view)[rows]
    bad = got != q_ref
    assert not bad.any(), "%d of %d codes differ; first %s" % (bad.sum(), bad.size, np.argwhere(bad)[:3])
    assert (np.abs(q_ref) == 127).any(), "the case should reach the clamp"


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("M,N,K", [(16, 256, 256), (300, 520, 384)])
def test_requant_with_activation(ql, act, M, N, K):
    """With an activation the kernel's act(y) differs from the oracle's fp64 act(y32) by the
    activation's error (about 1e-6 relative), so a code may differ by one only where the
    exact quotient lies that close to a rounding boundary; everywhere else codes agree."""
    inp, rows, xq, xs, wq, ws, s_out, y32 = _requant_case(ql, M, N, K, False, 1)
    yq = ql.gemm_w8a8_requant(xq, xs, wq, ws, dev(s_out), dev(inp.bias), act)
    code = {"gelu": 1, "silu": 2}[act]
    a = oracle.activation_f64(y32.astype(np.float64), code)
    v = a / s_out.astype(np.float64)[None, :]
    q_ref = np.clip(np.rint(v), -127, 127)
    got = host(yq)[rows].astype(np.float64)
    delta = (4e-6 * (np.abs(y32) + np.abs(a)) + 1e-30) / s_out.astype(np.float64)[None, :]
    near = np.abs(np.abs(v - np.floor(v)) - 0.5) <= delta
    assert np.all(np.abs(got - q_ref) <= 1)
    assert np.all((got == q_ref) | near), "codes differ away from a rounding boundary"
    assert near.sum() < 0.01 * near.size


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (1, 4096, 4096), (5, 17, 192), (16, 4096, 4096), (17, 300, 128),
                                   (33, 1000, 640), (48, 16, 4096), (64, 31, 64), (65, 300, 256),
                                   (96, 1000, 640), (100, 17, 64), (128, 2048, 4096), (129, 300, 256),
                                   (1, 11008, 4096), (16, 11008, 4096), (24, 10240, 640), (8, 16384, 192),
                                   (64, 11008, 4096), (8, 2000, 2880), (12, 4096, 1600), (20, 1000, 1472)])
def test_few_rows_int32(ql, M, N, K):
    """The few-row kernel takes M <= 8, or M <= 128 with M * N <= 256K and N <= 12288 (16
    columns per workgroup, K split over the waves, 16x16x64 matrix-core steps after a lane
    permutation). Its four wave shapes are all covered: eight waves on a ring of 4 steps (at most
    2 x CUs workgroups, M <= 8) or 2 steps (9 <= M <= 64), with wave step counts below, at and
    past the ring's depth (e.g. M = 8, K = 2880: 5 or 6 steps per wave; M = 20, K = 1472: 2 or 3);
    four waves of 16-step groups (more workgroups than that: N > 8192, e.g. M = 16, N = 11008;
    M = 24, N = 10240; M = 8, N = 16384); and eight waves of 4-step groups for five to eight row
    blocks (M = 65 .. 128). Accumulators bit for bit, with codes at the extremes, ragged N, one
    to 64 k-steps; M = 129 and M = 64, N = 11008 (past 256K) run on the 64 x 64 kernel."""
    rng = np.random.default_rng(M * 7919 + N + K)
    a = _rand_codes(rng, (M, K), -128)
    b = _rand_codes(rng, (N, K), -128)
    a[0, :] = -128
    b[-1, :] = -128
    g = Guarded((M, N), torch.int32)
    ql.gemm_w8a8_int32(dev(a), dev(b), acc=g.view)
    g.check()
    assert np.array_equal(host(g.view), oracle.gemm_i32(a, b))


@pytest.mark.parametrize("act", ["none", "gelu", "silu"])
@pytest.mark.parametrize("M,N,K,out", [(1, 4096, 4096, torch.float16), (16, 300, 256, torch.float32),
                                       (40, 1000, 1024, torch.float16), (64, 257, 192, torch.float32),
                                       (128, 600, 256, torch.float16)])
def test_few_rows_layer(ql, act, M, N, K, out):
    """The few-row kernel's epilogue (scales, bias, activation; fp32 and fp16) within the same
    bounds as the tile kernel's."""
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N)
    inp, (xq, xs, wq, ws), (xq_r, xs_r, wq_r, ws_r) = _layer(ql, w)
    g = Guarded((M, N), out)
    ql.gemm_w8a8_per_channel_act(xq, xs, wq, ws, dev(inp.bias), act, out, y=g.view)
    g.check()
    acc = oracle.gemm_i32(xq_r, wq_r)
    y64 = oracle.epilogue_w8a8(acc, xs_r, ws_r, inp.bias)[1]
    mag = np.abs(acc.astype(np.float64) * xs_r[:, None] * ws_r[None, :]) + np.abs(inp.bias)[None, :]
    code = {"none": 0, "gelu": 1, "silu": 2}[act]
    ref = oracle.activation_f64(y64, code)
    tol = (1.13 if code else 1.0) * 1e-5 * mag + (6e-6 * np.abs(ref) if code else 0.0)
    if out == torch.float16:
        tol = tol + f16_ulp(ref)
    y = host(g.view).astype(np.float64)
    assert np.all(np.abs(y - ref) <= tol)


@pytest.mark.parametrize("M,N,K", [(64, 4096, 256), (65, 4096, 256), (8, 14336, 192), (9, 14336, 192),
                                   (16, 11008, 128), (24, 11008, 128), (512, 4096, 256), (513, 4096, 256),
                                   (128, 11008, 320), (129, 11008, 320), (200, 3001, 576), (1024, 4096, 192),
                                   (1025, 4096, 192), (300, 7000, 320), (600, 9000, 192), (384, 14336, 128),
                                   (1536, 11008, 128)])
def test_kernel_switches_int32(ql, M, N, K):
    """Shapes on both sides of each switch between the three W8A8 kernels: few-row against
    64 x 64 tiles (M * N = 256K at N = 4096; M = 8 against 9 at N = 14336 > 12288; 16 against
    24 rows at N = 11008), 64 x 64 tiles against the tile kernel (M = 512 against 513 at
    N = 4096, where 64 x 64 tiles pass two rounds; M = 128 against 129 at N = 11008, the latter
    on 128 x 128 tiles), a ragged 64 x 64 case with a half-deep last stage, and the tile
    kernel's plans without big tiles on both sides of the switch from 128 x 128 to 128 x 192
    tiles (M = 1024 against 1025 at N = 4096: 256 tiles of 128 x 128 against 198 of 128 x 192,
    where 128 x 128 would make 288; ragged at M = 300, N = 7000 with a half-deep last stage;
    128 x 192 at M = 600, N = 9000 and M = 384, N = 14336), and big tiles followed by 128 x 192
    tiles (M = 1536, N = 11008: 252 big tiles, then 24 small ones over the last 256 columns).
    Accumulators bit for bit on rows sampled from every 64-row band."""
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = _rand_codes(rng, (M, K), -128)
    b = _rand_codes(rng, (N, K), -128)
    acc = host(ql.gemm_w8a8_int32(dev(a), dev(b)))
    rows = np.unique(np.concatenate([np.arange(0, M, 13), np.arange(max(0, M - 3), M)]))
    assert np.array_equal(acc[rows], oracle.gemm_i32(a[rows], b))


@pytest.mark.parametrize("act", ["none", "gelu"])
@pytest.mark.parametrize("M,N,K,out", [(200, 3001, 576, torch.float16), (300, 1000, 256, torch.float32),
                                       (40, 11008, 512, torch.float16), (600, 4096, 256, torch.float16),
                                       (300, 7000, 320, torch.float32)])
def test_mid_tile_layer(ql, act, M, N, K, out):
    """The 64 x 64 kernel's epilogue (ragged N with scalar stores, fp16 and fp32 output, a fused
    activation), and the tile kernel's on 128 x 128 tiles (M = 600, N = 4096; ragged M and N at
    300 x 7000): within the tile kernel's tolerances, and with act = none bit for bit the value
    the plain call gives."""
    w = workloads.with_shape(workloads.W8A8_PREFILL, M, K, N, seed=M + N)
    inp, (xq, xs, wq, ws), (xq_r, xs_r, wq_r, ws_r) = _layer(ql, w)
    g = Guarded((M, N), out)
    ql.gemm_w8a8_per_channel_act(xq, xs, wq, ws, dev(inp.bias), act, out, y=g.view)
    g.check()
    acc_ref = oracle.gemm_i32(xq_r, wq_r)
    y32, y64 = oracle.epilogue_w8a8(acc_ref, xs_r, ws_r, inp.bias)
    y = host(g.view).astype(np.float64)
    mag = np.abs(acc_ref.astype(np.float64) * xs_r[:, None] * ws_r[None, :]) + np.abs(inp.bias)[None, :]
    if act == "none":
        if out == torch.float32:
            assert np.all(np.abs(y - y64) <= 1e-5 * mag)
        else:
            ref16 = y32.astype(np.float16).astype(np.float64)
            assert np.all(np.abs(y - ref16) <= f16_ulp(ref16))
        plain = host(ql.gemm_w8a8_per_channel(xq, xs, wq, ws, dev(inp.bias), out))
        assert np.array_equal(plain.view(np.uint8), host(g.view).view(np.uint8))
    else:
        a64 = oracle.activation_f64(y64, ACT[act])
        if out == torch.float32:
            assert np.all(np.abs(y - a64) <= 1.2e-5 * mag + 6e-6 * np.abs(a64))
        else:
            ref16 = a64.astype(np.float16).astype(np.float64)
            assert np.all(np.abs(y - ref16) <= f16_ulp(ref16))


def _finite_fp16_values() -> np.ndarray:
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)].astype(np.float32)


@pytest.mark.parametrize("M,N,out,act", [(1, 63488, torch.float16, "gelu"),     # few-row kernel
                                         (100, 8192, torch.float16, "gelu"),    # mid-size M
                                         (200, 63488, torch.float16, "gelu"),   # tile kernel
                                         (1, 63488, torch.float16, "silu"),
                                         (100, 8192, torch.float16, "silu"),
                                         (200, 63488, torch.float16, "silu"),
                                         (1, 63488, torch.float32, "gelu"),
                                         (200, 63488, torch.float32, "gelu")])
def test_activation_over_fp16_domain(ql, M, N, out, act):
    """X = 0 with unit scales makes the epilogue's pre-activation value exactly the bias, so a
    bias holding every finite fp16 value (N = 63,488; an evenly spread 8,192 of them, both ends
    included, for the mid-size case) runs the kernels' activation over the whole fp16 domain on
    the hardware, in every row. fp16 outputs: within one fp16 step of the correctly rounded
    act(y), for GELU (the fp16-output tail) and SiLU. fp32 outputs (GELU only; SiLU's fp32
    exponential underflows to an exact zero below y = -88, where act(y) is a denormal-sized
    nonzero; test_fused_activation covers it): within 2e-7 |y| of y Phi(y), the 9e-8 |y| that test_gelu_tail pins for the
    degree-11 tail in an exactly rounded emulation, plus v_exp_f32's own error of about one
    ulp on a tail of at most 1/2."""
    vals = _finite_fp16_values()
    if N < vals.size:
        vals = vals[np.unique(np.linspace(0, vals.size - 1, N).round().astype(np.int64))]
    assert vals.size == N
    K = 64
    rng = np.random.default_rng(N + M)
    a = np.zeros((M, K), np.int8)
    b = _rand_codes(rng, (N, K))
    g = Guarded((M, N), out)
    ql.gemm_w8a8_per_channel_act(dev(a), dev(np.ones(M, np.float32)), dev(b), dev(np.ones(N, np.float32)),
                                 dev(vals), act, out, y=g.view)
    g.check()
    y = host(g.view).astype(np.float64)
    ref = oracle.activation_f64(vals.astype(np.float64), ACT[act])
    if out == torch.float16:
        ref16 = ref.astype(np.float16).astype(np.float64)
        assert np.all(np.abs(y - ref16[None, :]) <= f16_ulp(ref16)[None, :])
    else:
        assert np.all(np.abs(y - ref[None, :]) <= 2e-7 * np.abs(vals.astype(np.float64))[None, :])
