"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph around the library's calls) and
replayed: each replay against the eager result of the same inputs, bit for bit, with eager work
and synchronizations between replays. The library allocates nothing and records no memset (the
per-tensor quantizer clears its slot with a kernel), so its calls capture; the graph reads the
static input buffers' current contents at every replay."""
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


def _inputs(rng, M, K, N, Md, Nd, M4, N4):
    x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xd = rng.standard_normal((Md, K)).astype(np.float16)
    wd = (rng.standard_normal((Nd, K)) * 0.02).astype(np.float32)
    x4 = rng.standard_normal((M4, K)).astype(np.float16)
    w4 = (rng.standard_normal((N4, K)) * 0.02).astype(np.float32)
    return x, w, xd, wd, x4, w4


def test_path_replayed_in_a_graph(ql):
    """Per-row quantizer + W8A8 GEMM (600 x 1024 x 2000: 128 x 128 split-K tiles), per-tensor
    quantizer (three launches), W8A16 decode (1 row) and W4A16 (32 rows, groups of 128)."""
    rng = np.random.default_rng(21)
    M, K, N, Md, Nd, M4, N4 = 600, 1024, 2000, 1, 3000, 32, 2500
    x, w, xd, wd, x4, w4 = _inputs(rng, M, K, N, Md, Nd, M4, N4)
    wq, ws = ql.quantize_weight_per_channel(dev(w))
    q8, s8 = ql.quantize_weight_per_channel(dev(wd))
    p4, s4 = ql.quantize_weight_int4_grouped(dev(w4), 128)
    bias = dev((rng.standard_normal(N) * 0.1).astype(np.float32))
    # static inputs: the graph reads these buffers
    sx, sxd, sx4 = dev(x), dev(xd), dev(x4)

    def run():
        xq, xs = ql.quantize_per_row_int8(sx)
        y = ql.gemm_w8a8_per_channel(xq, xs, wq, ws, bias, torch.float16)
        tq, ts = ql.quantize_per_tensor_int8(sx)
        yd = ql.gemm_w8a16(sxd, q8, s8)
        y4 = ql.gemm_w4a16_grouped(sx4, p4, s4, 128)
        return xq, xs, y, tq, ts, yd, y4

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()
    for rep in range(3):
        nx, _, nxd, _, nx4, _ = _inputs(np.random.default_rng(100 + rep), M, K, N, Md, Nd, M4, N4)
        sx.copy_(dev(nx))
        sxd.copy_(dev(nxd))
        sx4.copy_(dev(nx4))
        ref = [host(t).copy() for t in run()]   # eager, on the same inputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            got = host(a)
            assert got.dtype == b.dtype and got.shape == b.shape
            assert np.array_equal(got.view(np.uint8), b.view(np.uint8)), "replay %d, output %d differs" % (rep, i)
