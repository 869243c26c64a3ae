"""Helpers shared by the GPU parity tests (device transfer, tolerances, guard bands)."""
import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def f16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of fp16 at |v| (the gap to the next larger-magnitude fp16 number)."""
    return np.spacing(np.abs(v.astype(np.float16))).astype(np.float64)


def check_wonly(y_gpu: np.ndarray, y64: np.ndarray, rel: float = 2e-3):
    """Weight-only outputs: |y - y64| <= rel * (|y64| + rms(y64)) elementwise. Returns
    (normwise relative error, max elementwise relative error) for reporting."""
    y = y_gpu.astype(np.float64)
    rms = float(np.sqrt(np.mean(y64 ** 2))) if y64.size else 0.0
    err = np.abs(y - y64)
    bound = rel * (np.abs(y64) + rms)
    bad = err > bound
    assert not bad.any(), "%d of %d outside tolerance; worst %s vs %s" % (
        bad.sum(), bad.size, y[bad][:4], y64[bad][:4])
    norm = float(np.linalg.norm(y - y64) / max(np.linalg.norm(y64), 1e-300))
    return norm, float((err / np.maximum(np.abs(y64), 1e-30)).max()) if y64.size else 0.0


class Guarded:
    """An output buffer with sentinel-filled guard bands before and after it, to detect
    writes outside [0, numel)."""

    PAD = 4096

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.shape = shape
        self.buf = torch.empty(self.n + 2 * self.PAD, dtype=dtype, device=DEV)
        if dtype.is_floating_point:
            self.buf.fill_(-7777.0)
        else:
            self.buf.fill_(-77)
        self.sentinel = self.buf[:1].clone()
        self.view = self.buf[self.PAD:self.PAD + self.n].view(shape)

    def check(self):
        b = self.buf.cpu()
        s = self.sentinel.cpu()
        assert torch.equal(b[:self.PAD], s.expand(self.PAD)), "write before the output"
        assert torch.equal(b[self.PAD + self.n:], s.expand(self.PAD)), "write after the output"
