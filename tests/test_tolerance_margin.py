"""The weight-only GPU tests accept |y - y64| <= 2e-3 (|y64| + rms(y64)). This checks on the
CPU, at the decode workloads' shapes, that one legitimate fp32 summation order (the oracle's
k-order fp32 sum), rounded to the fp16 output, sits well inside that bound: the tolerance
covers fp32 reordering and the fp16 rounding with margin, and is not loose enough to hide a
dropped block of K (which moves y by far more; see the one-hot tests)."""
import numpy as np

import oracle
import workloads

TOL = 2e-3


def _ratio(y16, y64):
    rms = float(np.sqrt(np.mean(y64 ** 2)))
    return float((np.abs(y16.astype(np.float64) - y64) / (np.abs(y64) + rms)).max())


def test_w8a16_fp32_order_within_tolerance():
    inp = workloads.draw(workloads.W8A16_DECODE)
    q, s = oracle.quant_weight_per_channel(inp.w_nk)
    y64 = oracle.w8a16_f64(inp.x, q, s)
    y16 = oracle.w8a16_f32seq(inp.x, q, s).astype(np.float16)
    r = _ratio(y16, y64)
    assert r < TOL / 4, r


def test_block_asym_fp32_order_within_tolerance():
    inp = workloads.draw(workloads.W8A16_BLOCK)
    q, s, z = oracle.quant_block_asym_u8(inp.w_nk, 64)
    y64 = oracle.w8a16_f64(inp.x, q, s, z, 64)
    y16 = oracle.w8a16_f32seq(inp.x, q, s, z, 64).astype(np.float16)
    r = _ratio(y16, y64)
    assert r < TOL / 4, r


def test_w4a16_fp32_order_within_tolerance():
    """On the first 1024 output columns of the W4A16 workload: int4 codes as int8 with the
    stored fp16 group scales (exact in fp32)."""
    inp = workloads.draw(workloads.W4A16_GROUP)
    w = inp.w_nk[:1024]
    packed, s16 = oracle.quant_int4_group(w, 128)
    codes = oracle.unpack_int4(packed, w.shape[1]).astype(np.int8)
    s32 = (s16.view(np.float16) if s16.dtype == np.uint16 else s16).astype(np.float32)
    y64 = oracle.w8a16_f64(inp.x, codes, s32, None, 128)
    y16 = oracle.w8a16_f32seq(inp.x, codes, s32, None, 128).astype(np.float16)
    r = _ratio(y16, y64)
    assert r < TOL / 4, r
