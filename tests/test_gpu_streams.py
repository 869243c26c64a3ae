"""Calls on two streams at once: the library keeps no state between calls and enqueues its work
on the caller's stream, so two streams running the whole path concurrently on different inputs
give, bit for bit, what each gives alone."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    import int8_quantized_linear_amd as ql

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ql


def _case(ql, seed):
    """Inputs and weights of one stream's path: per-row quantizer, W8A8 GEMM at M2048 K4096
    N4096 (the tile kernel), per-tensor quantizer, W8A16 decode, block-asymmetric decode and
    W4A16 decode."""
    rng = np.random.default_rng(seed)
    M, K, N = 2048, 4096, 4096
    x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xd = rng.standard_normal((8, K)).astype(np.float16)
    wq, ws = ql.quantize_weight_per_channel(dev(w))
    qb, sb, zb = ql.quantize_weight_block_asym_u8(dev(w), 64)
    p4, s4 = ql.quantize_weight_int4_grouped(dev(w), 128)
    bias = dev((rng.standard_normal(N) * 0.1).astype(np.float32))
    return dict(x=dev(x), xd=dev(xd), wq=wq, ws=ws, qb=qb, sb=sb, zb=zb, p4=p4, s4=s4, bias=bias)


def _run(ql, c):
    xq, xs = ql.quantize_per_row_int8(c["x"])
    y = ql.gemm_w8a8_per_channel(xq, xs, c["wq"], c["ws"], c["bias"], torch.float16)
    tq, ts = ql.quantize_per_tensor_int8(c["x"])
    yd = ql.gemm_w8a16(c["xd"][:1], c["wq"], c["ws"])
    yb = ql.gemm_w8a16(c["xd"], c["qb"], c["sb"], c["zb"], 64)
    y4 = ql.gemm_w4a16_grouped(c["xd"], c["p4"], c["s4"], 128)
    return xq, xs, y, tq, ts, yd, yb, y4


def test_two_streams_concurrently(ql):
    cases = [_case(ql, 31), _case(ql, 32)]
    torch.cuda.synchronize()
    ref = [[host(t) for t in _run(ql, c)] for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [None, None]
    for _ in range(4):   # the calls of the two streams interleave as they are issued
        for i, (s, c) in enumerate(zip(streams, cases)):
            with torch.cuda.stream(s):
                outs[i] = _run(ql, c)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    names = ["xq", "xs", "y", "tq", "ts", "yd", "yb", "y4"]
    for i in range(2):
        for name, r, t in zip(names, ref[i], outs[i]):
            got = host(t)
            assert np.array_equal(got.view(np.uint8), r.view(np.uint8)), (i, name)
