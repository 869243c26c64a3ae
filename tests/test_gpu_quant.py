"""GPU parity of the quantizers against the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, Guarded, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    import int8_quantized_linear_amd as ql
    return ql


def _check_rows(ql, x: np.ndarray):
    q_ref, s_ref = oracle.quant_rows_i8(x)
    xq, xs = ql.quantize_per_row_int8(dev(x))
    assert np.array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(xq), q_ref)


def test_per_row_small_fp32(ql):
    _check_rows(ql, workloads.draw(workloads.W8A8_SMALL).x)


def test_per_row_prefill_full(ql):
    _check_rows(ql, workloads.draw(workloads.W8A8_PREFILL, x_rows=slice(0, 2048)).x)


@pytest.mark.parametrize("M,K,dtype", [(1, 16, np.float16), (37, 4096, np.float16),
                                       (5, 8256, np.float16), (3, 4112, np.float32),
                                       (64, 48, np.float32), (130, 1024, np.float16), (4, 11008, np.float16), (2, 14336, np.float16), (3, 16400, np.float16), (2, 8208, np.float32),
                                       (2, 1 << 20, np.float16), (1, 1 << 19, np.float32)])
def test_per_row_shapes(ql, M, K, dtype):
    """Ragged M, the shortest K, and rows too long to keep in registers."""
    rng = np.random.default_rng(M * 7 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, 1)))).astype(dtype)
    _check_rows(ql, x)


def test_per_row_special_rows(ql):
    """All-zero rows (absmax floor), a single nonzero, ties at scale 1, tiny values."""
    x = np.zeros((6, 64), np.float32)
    x[1, 9] = -3.0
    x[2, :12] = [127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -1.5, -126.5, 126.5, 0, -127]
    x[3, :] = 1e-30
    x[4, ::2] = 6e-8
    x[5, :] = np.linspace(-1, 1, 64)
    _check_rows(ql, x)


def test_per_row_fp16_domain(ql):
    """Every finite fp16 value as an activation, in rows with varied absmax."""
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(3)
    rng.shuffle(vals)
    K = 4096
    rows = -(-vals.size // K)
    x = np.zeros(rows * K, np.float16)
    x[:vals.size] = vals
    x = x.reshape(rows, K)
    _check_rows(ql, x)
    # the same values capped at several magnitudes
    for cap in (1.0, 127.0, 0.001):
        y = np.clip(x.astype(np.float32), -cap, cap).astype(np.float16)
        _check_rows(ql, y)


def test_per_row_guard_band(ql):
    x = np.random.default_rng(5).standard_normal((33, 4096)).astype(np.float16)
    g = Guarded((33, 4096), torch.int8)
    s = Guarded((33,), torch.float32)
    ql.quantize_per_row_int8(dev(x), g.view, s.view)
    g.check()
    s.check()
    q_ref, s_ref = oracle.quant_rows_i8(x)
    assert np.array_equal(host(g.view), q_ref)


def test_per_row_empty(ql):
    xq, xs = ql.quantize_per_row_int8(torch.empty((0, 64), dtype=torch.float16, device=DEV))
    assert xq.shape == (0, 64) and xs.shape == (0,)


@pytest.mark.parametrize("w", [workloads.W8A8_SMALL, workloads.W8A16_DECODE, workloads.W8A8_PREFILL],
                         ids=lambda w: w.name)
def test_weight_per_channel_full(ql, w):
    inp = workloads.draw(w, x_rows=slice(0, 1))
    q_ref, s_ref = oracle.quant_weight_per_channel(inp.w_nk)
    wq, ws = ql.quantize_weight_per_channel(dev(inp.w_nk))
    assert np.array_equal(host(ws).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(wq), q_ref)


@pytest.mark.parametrize("N,K,block", [(4096, 4096, 64), (77, 192, 64), (5, 256, 128), (3, 64, 16),
                                     (3, 1 << 20, 64)])
def test_block_asym_producer(ql, N, K, block):
    w = workloads.with_shape(workloads.W8A16_BLOCK, 1, K, N)
    inp = workloads.draw(w, x_rows=slice(0, 1))
    q_ref, s_ref, z_ref = oracle.quant_block_asym_u8(inp.w_nk, block)
    q, s, z = ql.quantize_weight_block_asym_u8(dev(inp.w_nk), block)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(z), z_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("N,K,group", [(14336, 4096, 128), (77, 384, 128), (9, 256, 64), (4, 64, 32),
                                     (2, 1 << 20, 128)])
def test_int4_producer(ql, N, K, group):
    w = workloads.with_shape(workloads.W4A16_GROUP, 1, K, N)
    inp = workloads.draw(w, x_rows=slice(0, 1))
    w_nk = inp.w_nk
    w_nk[0, :group] = 0.0                      # an all-zero group: the scale floor
    p_ref, s_ref = oracle.quant_int4_group(w_nk, group)
    p, s = ql.quantize_weight_int4_grouped(dev(w_nk), group)
    assert np.array_equal(host(s).view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(host(p), p_ref)


# ------------------------------------------------------------ asymmetric rows

def _check_asym(ql, x):
    q_ref, s_ref, z_ref = oracle.quant_rows_i8_asym(x)
    q, s, z = ql.quantize_per_row_int8_asym(dev(x))
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(z).view(np.uint32), z_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("M,K,dtype", [(1, 16, np.float32), (37, 4096, np.float16), (5, 8256, np.float16),
                                       (3, 4112, np.float32), (130, 1024, np.float16), (64, 48, np.float32), (4, 11008, np.float16), (2, 14336, np.float16), (3, 16400, np.float16), (2, 8208, np.float32),
                                       (2, 1 << 20, np.float16)])
def test_asym_rows_bit_exact(ql, M, K, dtype):
    """Codes, scales and float zero points bit for bit: offset and scaled normal rows,
    rows longer than the registers hold (re-read), fp16 and fp32 inputs."""
    rng = np.random.default_rng(M * 13 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, 1)))
         + rng.uniform(-4, 4, (M, 1))).astype(dtype)
    _check_asym(ql, x)


def test_asym_special_rows(ql):
    """Rows with minimum 0 (zero point -128), constant rows (scale floor), a single
    nonzero, all-negative rows, and ties of x / s + z at .5."""
    rng = np.random.default_rng(91)
    K = 256
    rows = [np.abs(rng.standard_normal(K)), np.full(K, 0.75), np.zeros(K), -np.abs(rng.standard_normal(K)) - 3,
            np.eye(1, K, 17)[0] * 5.0, (rng.integers(0, 256, K) * 0.125) - 3.0, np.arange(K) * 0.5]
    x = np.stack(rows).astype(np.float32)
    _check_asym(ql, x)
    _check_asym(ql, x.astype(np.float16))


def test_column_sums(ql):
    rng = np.random.default_rng(92)
    for N, K in [(1, 16), (77, 4096), (11008, 256), (300, 4112)]:
        wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
        assert np.array_equal(host(ql.weight_column_sums_i8(dev(wq))), oracle.column_sums_i8(wq))
    wq = np.full((3, 131008), -128, np.int8)
    assert np.all(host(ql.weight_column_sums_i8(dev(wq))) == -128 * 131008)


def _check_tensor(ql, x: np.ndarray, xq_out=None, xs_out=None):
    q_ref, s_ref = oracle.quant_tensor_i8(x)
    xq, xs = ql.quantize_per_tensor_int8(dev(x))
    assert np.array_equal(host(xs).view(np.uint32), np.array([s_ref], np.float32).view(np.uint32))
    assert np.array_equal(host(xq), q_ref)


@pytest.mark.parametrize("shape,dtype", [((16,), np.float32), ((3, 16), np.float16), ((16, 256), np.float32),
                                         ((1, 4112), np.float32), ((77, 48), np.float16),
                                         ((2048, 4096), np.float16), ((1000, 2064), np.float16)])
def test_per_tensor(ql, shape, dtype):
    """One scale for the whole array, bit for bit: sizes below one workgroup's step, ragged
    sizes, the prefill activations (more chunks than the grid covers in one step, so the
    grid-stride loops run several times) and fp16 and fp32 inputs."""
    rng = np.random.default_rng(int(np.prod(shape)) + 3)
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-5, 5))).astype(dtype)
    _check_tensor(ql, x)


def test_per_tensor_weights_full(ql):
    """The prefill weight [11008, 4096] fp32 with a single scale (the per-tensor baseline of
    the weight quantizer)."""
    _check_tensor(ql, workloads.draw(workloads.W8A8_PREFILL, x_rows=slice(0, 1)).w_nk)


def test_per_tensor_special(ql):
    """The maximum in the very last chunk; a negative maximum; an all-zero tensor (scale
    floor); -0; and a reused scale buffer that held a larger value before (it is cleared
    by the call, not folded into the new maximum)."""
    n = 2048 * 4096 + 16
    x = np.full(n, 0.25, np.float32)
    x[-1] = 3.0
    _check_tensor(ql, x)
    x[-1] = -5.0
    _check_tensor(ql, x)
    _check_tensor(ql, np.zeros(64, np.float32))
    z = np.full(32, -0.0, np.float16)
    z[7] = 1.0
    _check_tensor(ql, z)
    big = dev(np.full(64, 1000.0, np.float32))
    small = np.random.default_rng(9).standard_normal(4096).astype(np.float32)
    xq = torch.empty(4096, dtype=torch.int8, device=DEV)
    xs = torch.empty(1, dtype=torch.float32, device=DEV)
    xq64 = torch.empty(64, dtype=torch.int8, device=DEV)
    ql._call("quantize_per_tensor_int8", ql._ptr(big), 0, 64, ql._ptr(xq64), ql._ptr(xs), ql._stream(big))
    xd = dev(small)
    ql._call("quantize_per_tensor_int8", ql._ptr(xd), 0, 4096, ql._ptr(xq), ql._ptr(xs), ql._stream(xd))
    q_ref, s_ref = oracle.quant_tensor_i8(small)
    assert host(xs)[0] == np.float32(s_ref) and np.array_equal(host(xq), q_ref)
