"""Parity on seeded random shapes, every path, each case reproducible from its seed.

Shapes are drawn within each entry point's stated requirements (K a multiple of 64, block and
group sizes dividing K) with ragged M and N, so tile edges, partial k-stages and the
half-height, mixed and big tile plans are all hit across the draws. Inputs are normal with a
per-case scale. The bars are the other parity tests':
- int32 accumulators and int8-output codes bit for bit;
- fp8 sums exact on half-integer codes;
- weight-only outputs within 2e-3 (|y64| + rms(y64)).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, check_wonly, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    import int8_quantized_linear_amd as ql
    return ql


def _shape(seed, m_max, n_max, k_max):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, m_max + 1))
    N = int(rng.integers(1, n_max + 1))
    K = 64 * int(rng.integers(1, k_max // 64 + 1))
    return rng, M, N, K


@pytest.mark.parametrize("seed", range(1000, 1016))
def test_w8a8_int32_random(ql, seed):
    rng, M, N, K = _shape(seed, 700, 1500, 1024)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    g = Guarded((M, N), torch.int32)
    ql.gemm_w8a8_int32(dev(a), dev(b), acc=g.view)
    g.check()
    assert np.array_equal(host(g.view), oracle.gemm_i32(a, b)), (M, N, K)


def _large_shape(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(129, 4097))
    N = int(rng.integers(256, 16385))
    K = 64 * int(rng.integers(1, 9))
    return rng, M, N, K


def _sampled_rows(M):
    return np.unique(np.concatenate([np.arange(0, M, 97), np.arange(M - 3, M)]))


@pytest.mark.parametrize("seed", range(1100, 1124))
def test_w8a8_int32_random_tile_plans(ql, seed):
    """Large random shapes (M 129..4096, N 256..16384), where the routing takes every tile
    plan across the draws: 64 x 64 tiles, 128 x 128, 128 x 192 and 128 x 256 split-K tiles
    alone, big tiles alone (256 x 256 in one or several rounds, 256 x 192), and big tiles
    followed by 128 x 192 or 128 x 256 tiles. Accumulators bit for bit on rows sampled from
    every band of 97."""
    rng, M, N, K = _large_shape(seed)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    g = Guarded((M, N), torch.int32)
    ql.gemm_w8a8_int32(dev(a), dev(b), acc=g.view)
    g.check()
    rows = _sampled_rows(M)
    assert np.array_equal(host(g.view)[rows], oracle.gemm_i32(a[rows], b)), (M, N, K)


@pytest.mark.parametrize("seed", range(3100, 3106))
def test_e4m3_exact_random_tile_plans(ql, seed):
    """The fp8 layer on large random shapes (the same draws' plans), exact on half-integer
    codes, rows sampled from every band of 97."""
    rng, M, N, K = _large_shape(seed)
    table = oracle.e4m3_encode((np.arange(-15, 16) / 2).astype(np.float32))
    a = table[rng.integers(0, 31, (M, K))]
    b = table[rng.integers(0, 31, (N, K))]
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    y = ql.gemm_e4m3_per_channel(dev(a), dev(ones_m), dev(b), dev(ones_n), out_dtype=torch.float32)
    rows = _sampled_rows(M)
    y64, _ = oracle.gemm_e4m3_f64(a[rows], ones_m[rows], b, ones_n)
    assert np.array_equal(host(y)[rows].astype(np.float64), y64), (M, N, K)


@pytest.mark.parametrize("seed", range(2000, 2010))
def test_w8a8_requant_random(ql, seed):
    """Quantizers, GEMM and int8 output on random shapes, per-column or per-tensor scales."""
    rng, M, N, K = _shape(seed, 600, 1200, 768)
    x = (rng.standard_normal((M, K)) * rng.uniform(0.1, 10)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * rng.uniform(0.001, 0.1)).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
    xq_r, xs_r = oracle.quant_rows_i8(x)
    wq_r, ws_r = oracle.quant_weight_per_channel(w)
    xq, xs = ql.quantize_per_row_int8(dev(x))
    wq, ws = ql.quantize_weight_per_channel(dev(w))
    assert np.array_equal(host(xq), xq_r) and np.array_equal(host(wq), wq_r)
    y32 = oracle.epilogue_w8a8(oracle.gemm_i32(xq_r, wq_r), xs_r, ws_r, bias)[0]
    s_out = oracle.channel_scales(y32) * np.float32(0.8)
    if seed % 2:
        s_out = np.array([s_out.max()], np.float32)
    g = Guarded((M, N), torch.int8)
    ql.gemm_w8a8_requant(xq, xs, wq, ws, dev(s_out), dev(bias), "none", yq=g.view)
    g.check()
    assert np.array_equal(host(g.view), oracle.requant_i8(y32, s_out)), (M, N, K)


@pytest.mark.parametrize("seed", range(3000, 3008))
def test_e4m3_exact_random(ql, seed):
    rng, M, N, K = _shape(seed, 600, 1200, 1024)
    table = oracle.e4m3_encode((np.arange(-15, 16) / 2).astype(np.float32))
    a = table[rng.integers(0, 31, (M, K))]
    b = table[rng.integers(0, 31, (N, K))]
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    y = ql.gemm_e4m3_per_channel(dev(a), dev(ones_m), dev(b), dev(ones_n), out_dtype=torch.float32)
    y64, _ = oracle.gemm_e4m3_f64(a, ones_m, b, ones_n)
    assert np.array_equal(host(y).astype(np.float64), y64), (M, N, K)


@pytest.mark.parametrize("seed", range(4000, 4008))
def test_w8a16_random(ql, seed):
    rng, M, N, K = _shape(seed, 80, 1500, 2048)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s = oracle.quant_weight_per_channel(w)
    g = Guarded((M, N), torch.float16)
    ql.gemm_w8a16(dev(x), dev(q), dev(s), y=g.view)
    g.check()
    check_wonly(host(g.view), oracle.w8a16_f64(x, q, s))


@pytest.mark.parametrize("seed", range(5000, 5008))
def test_w8a16_block_random(ql, seed):
    rng, M, N, K = _shape(seed, 80, 1500, 2048)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02 + rng.uniform(-0.01, 0.01, (N, 1))).astype(np.float32)
    q, s, z = oracle.quant_block_asym_u8(w, 64)
    g = Guarded((M, N), torch.float16)
    ql.gemm_w8a16(dev(x), dev(q), dev(s), dev(z), 64, y=g.view)
    g.check()
    check_wonly(host(g.view), oracle.w8a16_f64(x, q, s, z, 64))


@pytest.mark.parametrize("seed", range(6000, 6008))
def test_w4a16_random(ql, seed):
    rng, M, N, K = _shape(seed, 80, 1500, 2048)
    group = 128 if (K % 128 == 0 and seed % 2 == 0) else 64
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    p, s16 = oracle.quant_int4_group(w, group)
    g = Guarded((M, N), torch.float16)
    ql.gemm_w4a16_grouped(dev(x), dev(p), dev(s16), group, y=g.view)
    g.check()
    check_wonly(host(g.view), oracle.w4a16_f64(x, p, s16, group))
