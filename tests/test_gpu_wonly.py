"""GPU parity of the weight-only paths (W8A16 per-channel, W8A16 block-asymmetric,
W4A16 per-group) against the oracle's fp64 products.

Tolerance: |y - y64| <= 2e-3 * (|y64| + rms(y64)) elementwise, with rms over the whole
output. fp16 output rounding alone is 2^-11 ~ 4.9e-4 of |y|; fp32 accumulation in any
order over K = 4096 terms adds well under that; a wrong code, nibble or scale index
moves outputs by O(rms).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, Guarded, check_wonly, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    import int8_quantized_linear_amd as ql
    return ql


def _w8a16_sym(ql, w: workloads.Workload, with_bias=False, group=0):
    inp = workloads.draw(w)
    bias = inp.bias if with_bias else None
    if with_bias and bias is None:
        bias = np.random.default_rng(w.seed).standard_normal(w.N).astype(np.float32) * 0.1
    q_ref, s_ref = oracle.quant_weight_per_channel(inp.w_nk)
    wq, ws = ql.quantize_weight_per_channel(dev(inp.w_nk))
    assert np.array_equal(host(wq), q_ref)
    g = Guarded((w.M, w.N), torch.float16)
    ql.gemm_w8a16(dev(inp.x), wq, ws, None, 0, dev(bias) if bias is not None else None, y=g.view)
    g.check()
    y64 = oracle.w8a16_f64(inp.x, q_ref, s_ref, bias=bias)
    return check_wonly(host(g.view), y64)


def test_w8a16_decode_full(ql):
    """M=1 K=4096 N=4096 decode GEMV, the benchmark's shape."""
    _w8a16_sym(ql, workloads.W8A16_DECODE)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 77, 192), (17, 1000, 640), (33, 130, 256),
                                   (70, 64, 128), (1, 9000, 256), (5, 8200, 128),
                                   (24, 9000, 512),    # 17..32 rows, 64-column tiles
                                   (3, 70, 1 << 20), (2, 17, 1 << 22)])   # long K, up to the largest allowed
def test_w8a16_ragged(ql, M, N, K):
    _w8a16_sym(ql, workloads.with_shape(workloads.W8A16_DECODE, M, K, N), with_bias=(M % 2 == 1))


def _w8a16_block(ql, w: workloads.Workload, block=64, with_bias=False):
    inp = workloads.draw(w)
    bias = (np.random.default_rng(w.seed).standard_normal(w.N) * 0.1).astype(np.float32) if with_bias else None
    q_ref, s_ref, z_ref = oracle.quant_block_asym_u8(inp.w_nk, block)
    q, s, z = ql.quantize_weight_block_asym_u8(dev(inp.w_nk), block)
    assert np.array_equal(host(q), q_ref) and np.array_equal(host(z), z_ref)
    g = Guarded((w.M, w.N), torch.float16)
    ql.gemm_w8a16(dev(inp.x), q, s, z, block, dev(bias) if bias is not None else None, y=g.view)
    g.check()
    y64 = oracle.w8a16_f64(inp.x, q_ref, s_ref, zero_point=z_ref, group_size=block, bias=bias)
    return check_wonly(host(g.view), y64)


def test_w8a16_block_full(ql):
    """M=8 K=4096 N=4096, blocks of 64 along K with uint8 zero points."""
    _w8a16_block(ql, workloads.W8A16_BLOCK)


@pytest.mark.parametrize("M,N,K,block", [(1, 50, 128, 64), (8, 333, 512, 128), (20, 100, 384, 192),
                                         (40, 9000, 128, 64), (3, 64, 256, 256),
                                         (24, 9000, 256, 64),    # one step in flight
                                         (56, 300, 256, 64),     # four row blocks
                                         (8, 40, 1 << 19, 64)])  # 8192 blocks a column: scales from global memory
def test_w8a16_block_ragged(ql, M, N, K, block):
    _w8a16_block(ql, workloads.with_shape(workloads.W8A16_BLOCK, M, K, N), block, with_bias=True)


def _w4a16(ql, w: workloads.Workload, group=128, with_bias=False, cols=None):
    inp = workloads.draw(w)
    bias = (np.random.default_rng(w.seed).standard_normal(w.N) * 0.1).astype(np.float32) if with_bias else None
    p_ref, s_ref = oracle.quant_int4_group(inp.w_nk, group)
    p, s = ql.quantize_weight_int4_grouped(dev(inp.w_nk), group)
    assert np.array_equal(host(p), p_ref)
    assert np.array_equal(host(s).view(np.uint16), s_ref.view(np.uint16))
    g = Guarded((w.M, w.N), torch.float16)
    ql.gemm_w4a16_grouped(dev(inp.x), p, s, group, dev(bias) if bias is not None else None, y=g.view)
    g.check()
    y = host(g.view)
    if cols is None:
        cols = np.arange(w.N)
    y64 = oracle.w4a16_f64(inp.x, p_ref[cols], s_ref[cols], group,
                           bias=None if bias is None else bias[cols])
    # rms of the full output is approximated by the sampled columns' rms
    return check_wonly(y[:, cols], y64)


def test_w4a16_full(ql):
    """M=32 K=4096 N=14336, group 128: every output against the oracle."""
    _w4a16(ql, workloads.W4A16_GROUP)


@pytest.mark.parametrize("M,N,K,group", [(1, 1, 128, 128), (3, 77, 256, 128), (32, 1000, 512, 64),
                                         (17, 9000, 256, 256), (65, 96, 384, 128), (8, 70, 128, 64),
                                         (24, 9000, 512, 64),    # 64-deep steps, one in flight
                                         (33, 50, 1 << 20, 128)])  # long K
def test_w4a16_ragged(ql, M, N, K, group):
    _w4a16(ql, workloads.with_shape(workloads.W4A16_GROUP, M, K, N), group, with_bias=True)


@pytest.mark.parametrize("fmt,M,N,K,group", [
    ("u8", 8, 16384, 4096, 64),     # 64 columns x 64 blocks (20 KB): staged, one row block
    ("u8", 20, 16384, 4096, 64),    # the same, staged at 17..32 rows
    ("u8", 40, 16384, 4096, 64),    # the same, staged at 33..48 rows (three row blocks)
    ("u8", 56, 16384, 4096, 64),    # the same over the 16 KB staging of 49..64 rows
    ("u8", 8, 16384, 8192, 64),     # 64 columns x 128 blocks (40 KB): over LDS at one row block
    ("i8", 20, 16384, 8192, 64),    # int8 with group scales, 64 x 128 fp32 scales: over LDS
    ("int4", 40, 3000, 1024, 64),   # 33..64 rows with 64-deep int4 steps
])
def test_large_scale_blocks_and_row_tiles(ql, fmt, M, N, K, group):
    """Plans whose scale block is too large for LDS (scales and zero points loaded from
    global memory every step, beside the activation ring) or only fits the larger staging
    area of one row block, and four row tiles with 64-deep int4 steps. Codes, scales and
    zero points are drawn directly (the quantizers have tests of their own)."""
    if fmt == "int4":
        _w4a16(ql, workloads.with_shape(workloads.W4A16_GROUP, M, K, N, seed=M + N), group,
               with_bias=True, cols=np.arange(0, N, 7))
        return
    w = workloads.with_shape(workloads.W8A16_DECODE, M, K, N, seed=M + N)
    inp = workloads.draw(w)
    rng = np.random.default_rng(M * N + K)
    s_ref = rng.uniform(1e-3, 1e-2, (N, K // group)).astype(np.float32)
    g = Guarded((M, N), torch.float16)
    if fmt == "u8":
        q_ref = rng.integers(0, 256, (N, K), dtype=np.uint8)
        z_ref = rng.integers(0, 256, (N, K // group), dtype=np.uint8)
        bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
        ql.gemm_w8a16(dev(inp.x), dev(q_ref), dev(s_ref), dev(z_ref), group, dev(bias), y=g.view)
        g.check()
        y64 = oracle.w8a16_f64(inp.x, q_ref, s_ref, zero_point=z_ref, group_size=group, bias=bias)
    else:
        q_ref = rng.integers(-127, 128, (N, K), dtype=np.int8)
        ql.gemm_w8a16(dev(inp.x), dev(q_ref), dev(s_ref), None, group, None, y=g.view)
        g.check()
        y64 = oracle.w8a16_f64(inp.x, q_ref, s_ref, group_size=group)
    check_wonly(host(g.view), y64)


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("M,N,K,group", [(32, 14336, 4096, 128), (3, 77, 256, 128), (40, 1000, 512, 64)])
def test_w4a16_fused_activation(ql, act, M, N, K, group):
    """act(W4A16 + bias) from the decode epilogue ([xdnf] §8), against the oracle's fp64
    activation of its fp64 product: the weight-only bound 2e-3 (|y64| + rms) on the
    pre-activation value, times max |act'| = 1.13 (the fp16 rounding of act(y) is within
    it since |act(y)| <= |y|). The full decode shape is checked on sampled columns."""
    code = {"gelu": 1, "silu": 2}[act]
    w = workloads.with_shape(workloads.W4A16_GROUP, M, K, N, seed=M + N + code)
    inp = workloads.draw(w)
    rng = np.random.default_rng(M + N)
    bias = (rng.standard_normal(N) * 0.5).astype(np.float32)
    p_ref, s_ref = oracle.quant_int4_group(inp.w_nk, group)
    p, s = ql.quantize_weight_int4_grouped(dev(inp.w_nk), group)
    g = Guarded((M, N), torch.float16)
    ql.gemm_w4a16_grouped_act(dev(inp.x), p, s, group, dev(bias), act, y=g.view)
    g.check()
    cols = np.arange(N) if N <= 2000 else np.unique(np.concatenate([np.arange(0, N, 13), np.arange(N - 40, N)]))
    y64 = oracle.w4a16_f64(inp.x, p_ref[cols], s_ref[cols], group, bias=bias[cols])
    ref = oracle.activation_f64(y64, code)
    y = host(g.view)[:, cols].astype(np.float64)
    rms = float(np.sqrt(np.mean(y64 ** 2)))
    assert np.all(np.abs(y - ref) <= 1.13 * 2e-3 * (np.abs(y64) + rms))


@pytest.mark.parametrize("N", [40, 10240])   # 8-column and 40-column workgroups (one and four column blocks)
def test_one_hot_exact(ql, N):
    """x = e_k: the group sums are exact (one product of an exact integer weight and 1.0), so
    y[n] is fp16(fp32((q[k,n] - z) * s)) exactly for all three formats: the scale multiplies the
    sum once in fp32 and the result is rounded once more to fp16. (For int8 codes the fp32
    product is not always exact, and rounding twice differs from rounding fp64 (q - z) * s
    straight to fp16 in a few elements of 70,000.)"""
    K = 256
    rng = np.random.default_rng(17)
    ks = [0, 7, 8, 63, 64, 130, 255]
    x = np.zeros((len(ks), K), np.float16)
    x[np.arange(len(ks)), ks] = 1.0
    w = rng.standard_normal((N, K)).astype(np.float32)

    def f32_then_f16(q, s):
        return (np.asarray(q, np.float32) * np.asarray(s, np.float32)).astype(np.float16)

    q_ref, s_ref = oracle.quant_weight_per_channel(w)
    wq, ws = ql.quantize_weight_per_channel(dev(w))
    y = host(ql.gemm_w8a16(dev(x), wq, ws))
    assert np.array_equal(y, f32_then_f16(q_ref[:, ks].T, s_ref[None, :]))
    qb, sb, zb = oracle.quant_block_asym_u8(w, 64)
    q, s, z = ql.quantize_weight_block_asym_u8(dev(w), 64)
    y = host(ql.gemm_w8a16(dev(x), q, s, z, 64))
    ref = np.stack([f32_then_f16(qb[:, k].astype(np.int32) - zb[:, k // 64], sb[:, k // 64]) for k in ks])
    assert np.array_equal(y, ref)
    p_ref, s16 = oracle.quant_int4_group(w, 128)
    p, s = ql.quantize_weight_int4_grouped(dev(w), 128)
    y = host(ql.gemm_w4a16_grouped(dev(x), p, s, 128))
    qi = oracle.unpack_int4(p_ref, K)
    ref = np.stack([f32_then_f16(qi[:, k], s16[:, k // 128].astype(np.float32)) for k in ks])
    assert np.array_equal(y, ref)


def test_empty(ql):
    x = torch.empty((0, 64), dtype=torch.float16, device=DEV)
    wq = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    y = ql.gemm_w8a16(x, wq, torch.ones(8, device=DEV))
    assert y.shape == (0, 8)


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("M", [1, 32])
def test_w4a16_activation_over_fp16_domain(ql, act, M):
    """X = 0 makes the decode epilogue's pre-activation value exactly the bias, so a bias
    holding every finite fp16 value (N = 63,488) runs the W4A16 epilogue's activation over the
    whole fp16 domain on the hardware, in every row: within one fp16 step of the correctly
    rounded act(y) (GELU through the fp16-output tail)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = h[np.isfinite(h)].astype(np.float32)
    N, K, group = vals.size, 128, 128
    rng = np.random.default_rng(M)
    w_nk = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    p, s = ql.quantize_weight_int4_grouped(dev(w_nk), group)
    g = Guarded((M, N), torch.float16)
    ql.gemm_w4a16_grouped_act(dev(np.zeros((M, K), np.float16)), p, s, group, dev(vals), act, y=g.view)
    g.check()
    y = host(g.view).astype(np.float64)
    ref = oracle.activation_f64(vals.astype(np.float64), {"gelu": 1, "silu": 2}[act])
    ref16 = ref.astype(np.float16).astype(np.float64)
    step = np.spacing(np.abs(ref.astype(np.float16))).astype(np.float64)
    assert np.all(np.abs(y - ref16[None, :]) <= step[None, :])
