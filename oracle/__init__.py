"""CPU oracle for the symmetric per-channel quantized linear layer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the HIP library and its
Python binding never do. The arithmetic lives in ``ql_oracle.c`` (plain loops,
built with gcc ``-O2 -fopenmp -ffp-contract=off -fno-fast-math``); this file only
moves numpy arrays in and out of it.

fp16 arrays cross into C as their binary16 bit patterns and are decoded there by
the oracle's own binary16 routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ql_oracle.c")
_HDR = os.path.join(_HERE, "ql_oracle.h")
_LIB = os.path.join(_HERE, "libqloracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
          "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (CPU only). Returns the library path."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _declare(L):
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f32.restype = ctypes.c_float
    L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_f16_to_f32_array.argtypes = [_P, _I64, _P]
    L.oracle_f32_to_f16_array.argtypes = [_P, _I64, _P]
    L.oracle_quant_rows_i8.argtypes = [_P, _I64, _I64, _P, _P]
    L.oracle_quant_tensor_i8.argtypes = [_P, _I64, _P]
    L.oracle_quant_tensor_i8.restype = ctypes.c_float
    L.oracle_gemm_i32.argtypes = [_P, _P, _I64, _I64, _I64, _P]
    L.oracle_gemm_i32.restype = ctypes.c_int
    L.oracle_epilogue_w8a8.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P]
    L.oracle_wonly_f64.argtypes = [_P, _I64, _I64, _P, ctypes.c_int, _P, _P, _I64, _P, _I64, _P]
    L.oracle_w4a16_f64.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _I64, _P]
    L.oracle_unpack_int4.argtypes = [_P, _I64, _I64, _P]
    L.oracle_quant_block_asym_u8.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
    L.oracle_quant_int4_group.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_activation_f64.argtypes = [_P, _I64, ctypes.c_int]
    L.oracle_quant_rows_i8_asym.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.oracle_channel_scales.argtypes = [_P, _I64, _I64, _P]
    L.oracle_wonly_f32seq.argtypes = [_P, _I64, _I64, _P, ctypes.c_int, _P, _P, _I64, _P, _I64, _P]
    L.oracle_requant_i8.argtypes = [_P, _I64, _I64, _P, _I64, _P]
    L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_decode.restype = ctypes.c_double
    L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_quant_rows_e4m3.argtypes = [_P, _I64, _I64, _P, _P]
    L.oracle_gemm_e4m3_f64.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
    L.oracle_column_sums_i8.argtypes = [_P, _I64, _I64, _P]
    L.oracle_w8a8_asym_f64.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """The oracle's functions bound to one compiled copy of ql_oracle.c."""

    def __init__(self, path: str):
        self.path = path
        self.L = ctypes.CDLL(path)
        _declare(self.L)

    # ----------------------------------------------------------------- binary16

    def f16_bits_to_f32(self, bits: np.ndarray) -> np.ndarray:
        bits = _c(bits, np.uint16)
        out = np.empty(bits.shape, np.float32)
        self.L.oracle_f16_to_f32_array(_ptr(bits), bits.size, _ptr(out))
        return out

    def f32_to_f16_bits(self, x: np.ndarray) -> np.ndarray:
        x = _c(x, np.float32)
        out = np.empty(x.shape, np.uint16)
        self.L.oracle_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
        return out

    def _as_f32(self, x: np.ndarray) -> np.ndarray:
        """fp16 activations are decoded by the oracle's own binary16 routine; fp32 pass through."""
        if x.dtype == np.float16:
            return self.f16_bits_to_f32(x.view(np.uint16))
        return _c(x, np.float32)

    # -------------------------------------------------------- symmetric int8

    def quant_rows_i8(self, x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Per-row symmetric int8 of a [rows, cols] array: (q int8 [rows, cols], scale fp32 [rows])."""
        xf = self._as_f32(x)
        rows, cols = xf.shape
        q = np.empty((rows, cols), np.int8)
        s = np.empty(rows, np.float32)
        self.L.oracle_quant_rows_i8(_ptr(xf), rows, cols, _ptr(q), _ptr(s))
        return q, s

    def quant_weight_per_channel(self, w_nk: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Per-output-channel symmetric int8 of W [K, N] column-major (given as [N, K])."""
        return self.quant_rows_i8(w_nk)

    def quant_tensor_i8(self, x: np.ndarray) -> Tuple[np.ndarray, float]:
        xf = self._as_f32(x)
        q = np.empty(xf.shape, np.int8)
        s = self.L.oracle_quant_tensor_i8(_ptr(xf), xf.size, _ptr(q))
        return q, float(np.float32(s))

    # -------------------------------------------------------------- W8A8

    def gemm_i32(self, xq: np.ndarray, wq_nk: np.ndarray) -> np.ndarray:
        xq = _c(xq, np.int8)
        wq_nk = _c(wq_nk, np.int8)
        M, K = xq.shape
        N, K2 = wq_nk.shape
        assert K == K2
        acc = np.empty((M, N), np.int32)
        bad = self.L.oracle_gemm_i32(_ptr(xq), _ptr(wq_nk), M, N, K, _ptr(acc))
        if bad:
            raise OverflowError("integer GEMM left the int32 range")
        return acc

    def epilogue_w8a8(self, acc, x_scale, w_scale, bias=None) -> Tuple[np.ndarray, np.ndarray]:
        acc = _c(acc, np.int32)
        xs = _c(x_scale, np.float32)
        ws = _c(w_scale, np.float32)
        b = None if bias is None else _c(bias, np.float32)
        M, N = acc.shape
        y32 = np.empty((M, N), np.float32)
        y64 = np.empty((M, N), np.float64)
        self.L.oracle_epilogue_w8a8(_ptr(acc), _ptr(xs), _ptr(ws), _ptr(b), M, N, _ptr(y32), _ptr(y64))
        return y32, y64

    def linear_w8a8(self, x, wq_nk, w_scale, bias=None):
        """Whole W8A8 layer: per-row quantization of x, int32 GEMM, fp32/fp64 epilogue.
        Returns dict(xq, x_scale, acc, y32, y64)."""
        xq, xs = self.quant_rows_i8(x)
        acc = self.gemm_i32(xq, wq_nk)
        y32, y64 = self.epilogue_w8a8(acc, xs, w_scale, bias)
        return dict(xq=xq, x_scale=xs, acc=acc, y32=y32, y64=y64)

    # ------------------------------------------------------------ weight-only

    def w8a16_f64(self, x, codes_nk, scale, zero_point=None, group_size: int = 0, bias=None) -> np.ndarray:
        """fp64 weight-only product. int8 codes (symmetric, zero_point None) or uint8 codes
        with zero points; scale [N] (group_size 0) or [N, K/group] (col-major [K/group, N])."""
        xf = self._as_f32(x)
        M, K = xf.shape
        N = codes_nk.shape[0]
        kind = 0 if zero_point is None else 1
        codes = _c(codes_nk, np.int8 if kind == 0 else np.uint8)
        s = _c(scale, np.float32)
        z = None if zero_point is None else _c(zero_point, np.uint8)
        b = None if bias is None else _c(bias, np.float32)
        y64 = np.empty((M, N), np.float64)
        self.L.oracle_wonly_f64(_ptr(xf), M, K, _ptr(codes), kind, _ptr(s), _ptr(z), group_size,
                               _ptr(b), N, _ptr(y64))
        return y64

    def w8a16_f32seq(self, x, codes_nk, scale, zero_point=None, group_size: int = 0, bias=None) -> np.ndarray:
        """The weight-only product of w8a16_f64 summed in fp32 in k order (one fp32 order)."""
        xf = self._as_f32(x)
        M, K = xf.shape
        N = codes_nk.shape[0]
        kind = 0 if zero_point is None else 1
        codes = _c(codes_nk, np.int8 if kind == 0 else np.uint8)
        s = _c(scale, np.float32)
        z = None if zero_point is None else _c(zero_point, np.uint8)
        b = None if bias is None else _c(bias, np.float32)
        y32 = np.empty((M, N), np.float32)
        self.L.oracle_wonly_f32seq(_ptr(xf), M, K, _ptr(codes), kind, _ptr(s), _ptr(z), group_size,
                                  _ptr(b), N, _ptr(y32))
        return y32

    def quant_rows_i8_asym(self, x) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Asymmetric int8 per row of x [M, K] (fp16 or fp32): (q int8, scale fp32 [M],
        zero fp32 [M]) with x ~ scale * (q - zero)."""
        xf = self._as_f32(x)
        M, K = xf.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        z = np.empty(M, np.float32)
        self.L.oracle_quant_rows_i8_asym(_ptr(xf), M, K, _ptr(q), _ptr(s), _ptr(z))
        return q, s, z

    def column_sums_i8(self, wq_nk) -> np.ndarray:
        """int32 [N]: the sum of each column's codes (W stored [N][K])."""
        w = _c(wq_nk, np.int8)
        N, K = w.shape
        out = np.empty(N, np.int32)
        self.L.oracle_column_sums_i8(_ptr(w), N, K, _ptr(out))
        return out

    def w8a8_asym_f64(self, xq, x_scale, x_zero, wq_nk, w_scale, bias=None) -> np.ndarray:
        """fp64 layer output with asymmetric activations, from the definition."""
        xq = _c(xq, np.int8)
        wq = _c(wq_nk, np.int8)
        M, K = xq.shape
        N = wq.shape[0]
        xs, xz, ws = _c(x_scale, np.float32), _c(x_zero, np.float32), _c(w_scale, np.float32)
        b = None if bias is None else _c(bias, np.float32)
        y64 = np.empty((M, N), np.float64)
        self.L.oracle_w8a8_asym_f64(_ptr(xq), _ptr(xs), _ptr(xz), _ptr(wq), _ptr(ws), _ptr(b), M, N, K,
                                    _ptr(y64))
        return y64

    def channel_scales(self, y) -> np.ndarray:
        """fp32 [N]: calibrated static scales max(max_m |y[m, n]|, 1e-10) / 127 of y [M, N]."""
        yf = _c(y, np.float32)
        M, N = yf.shape
        s = np.empty(N, np.float32)
        self.L.oracle_channel_scales(_ptr(yf), M, N, _ptr(s))
        return s

    def requant_i8(self, y, scale) -> np.ndarray:
        """int8 [M, N]: clamp(rne(y / scale[n]), -127, 127) of fp32 y [M, N]; scale has N
        entries (per channel) or one (per tensor)."""
        yf = _c(y, np.float32)
        M, N = yf.shape
        sc = _c(np.atleast_1d(scale), np.float32)
        if sc.size not in (1, N):
            raise ValueError("scale must have 1 or N entries")
        q = np.empty((M, N), np.int8)
        self.L.oracle_requant_i8(_ptr(yf), M, N, _ptr(sc), sc.size, _ptr(q))
        return q

    def e4m3_decode(self, codes) -> np.ndarray:
        """fp64 values of OCP e4m3 codes (NaN for S.1111.111)."""
        c = np.asarray(codes, np.uint8)
        return np.array([self.L.oracle_e4m3_decode(int(v)) for v in c.ravel()]).reshape(c.shape)

    def e4m3_encode(self, x) -> np.ndarray:
        """e4m3 codes of fp32 values with |x| <= 448, nearest, ties to even."""
        a = np.asarray(x, np.float32)
        return np.array([self.L.oracle_e4m3_encode(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)

    def quant_rows_e4m3(self, x) -> Tuple[np.ndarray, np.ndarray]:
        """Per-row fp8 of x [M, K] (fp16 or fp32): (codes uint8 [M, K], scale fp32 [M])."""
        xf = self._as_f32(x)
        M, K = xf.shape
        q = np.empty((M, K), np.uint8)
        s = np.empty(M, np.float32)
        self.L.oracle_quant_rows_e4m3(_ptr(xf), M, K, _ptr(q), _ptr(s))
        return q, s

    def gemm_e4m3_f64(self, xq, x_scale, wq_nk, w_scale, bias=None) -> Tuple[np.ndarray, np.ndarray]:
        """(y64, mag): the fp8 layer in fp64, and x_scale w_scale sum_k |products|."""
        xq = _c(xq, np.uint8)
        wq = _c(wq_nk, np.uint8)
        M, K = xq.shape
        N = wq.shape[0]
        xs, ws = _c(x_scale, np.float32), _c(w_scale, np.float32)
        b = None if bias is None else _c(bias, np.float32)
        y64 = np.empty((M, N), np.float64)
        mag = np.empty((M, N), np.float64)
        self.L.oracle_gemm_e4m3_f64(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(b), M, N, K, _ptr(y64), _ptr(mag))
        return y64, mag

    ACT_NONE, ACT_GELU, ACT_SILU = 0, 1, 2

    def activation_f64(self, y, act: int) -> np.ndarray:
        """The epilogue's activation of an fp64 output, elementwise: 1 = GELU (exact,
        y * Phi(y)), 2 = SiLU (y * sigmoid(y)), 0 = none. Returns a new array."""
        out = np.array(y, dtype=np.float64, order="C", copy=True)
        self.L.oracle_activation_f64(_ptr(out), out.size, int(act))
        return out

    def w4a16_f64(self, x, packed_nk8, scale16, group_size: int, bias=None) -> np.ndarray:
        """fp64 W4A16 product; scale16 is fp16 (or its uint16 bits) [N, K/group]."""
        xf = self._as_f32(x)
        M, K = xf.shape
        N = packed_nk8.shape[0]
        p = _c(packed_nk8, np.int32)
        sb = _c(scale16.view(np.uint16) if scale16.dtype == np.float16 else scale16, np.uint16)
        b = None if bias is None else _c(bias, np.float32)
        y64 = np.empty((M, N), np.float64)
        self.L.oracle_w4a16_f64(_ptr(xf), M, K, _ptr(p), _ptr(sb), group_size, _ptr(b), N, _ptr(y64))
        return y64

    def unpack_int4(self, packed_nk8: np.ndarray, K: int) -> np.ndarray:
        p = _c(packed_nk8, np.int32)
        N = p.shape[0]
        q = np.empty((N, K), np.int8)
        self.L.oracle_unpack_int4(_ptr(p), N, K, _ptr(q))
        return q

    def quant_block_asym_u8(self, w_nk, block: int):
        """(q uint8 [N, K], scale fp32 [N, K/block], zero_point uint8 [N, K/block])."""
        w = _c(w_nk, np.float32)
        N, K = w.shape
        G = K // block
        q = np.empty((N, K), np.uint8)
        s = np.empty((N, G), np.float32)
        z = np.empty((N, G), np.uint8)
        self.L.oracle_quant_block_asym_u8(_ptr(w), N, K, block, _ptr(q), _ptr(s), _ptr(z))
        return q, s, z

    def quant_int4_group(self, w_nk, group: int):
        """(packed int32 [N, K/8], scale fp16 [N, K/group])."""
        w = _c(w_nk, np.float32)
        N, K = w.shape
        packed = np.empty((N, K // 8), np.int32)
        s16 = np.empty((N, K // group), np.uint16)
        self.L.oracle_quant_int4_group(_ptr(w), N, K, group, _ptr(packed), _ptr(s16))
        return packed, s16.view(np.float16)

    def num_threads(self) -> int:
        return int(self.L.oracle_num_threads())


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def __getattr__(name):
    # module-level access (oracle.quant_rows_i8, ...) goes to the default build
    if name.startswith("__"):
        raise AttributeError(name)
    return getattr(default(), name)
