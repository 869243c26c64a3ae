"""The C-ABI library on a machine without a GPU: it loads, exports every function that
include/ql.h declares, and rejects bad arguments with the documented status codes
before making any HIP call (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ql.h")
LIB = os.path.join(ROOT, "int8_quantized_linear_amd", "libql.so")

OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4
F32, F16 = 0, 1
A = 0x10000            # a fake, 16-byte aligned address: never dereferenced on error paths
MIS = 0x10001          # a misaligned one


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**([a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libql.so not built")
    L = ctypes.CDLL(LIB)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "quantize_per_row_int8": [P, I, I64, I64, P, P, P],
        "quantize_weight_per_channel": [P, I64, I64, P, P, P],
        "gemm_w8a8_per_channel": [P, P, P, P, P, P, I, I64, I64, I64, P],
        "gemm_w8a8_int32": [P, P, P, I64, I64, I64, P],
        "gemm_w8a16": [P, P, P, P, I64, P, P, I64, I64, I64, P],
        "gemm_w4a16_grouped": [P, P, P, I64, P, P, I64, I64, I64, P],
        "gemm_w8a8_per_channel_act": [P, P, P, P, P, I, P, I, I64, I64, I64, P],
        "gemm_w4a16_grouped_act": [P, P, P, I64, P, I, P, I64, I64, I64, P],
        "quantize_per_row_int8_asym": [P, I, I64, I64, P, P, P, P],
        "weight_column_sums_i8": [P, I64, I64, P, P],
        "gemm_w8a8_asym": [P, P, P, P, P, P, P, I, P, I, I64, I64, I64, P],
        "quantize_per_row_e4m3": [P, I, I64, I64, P, P, P],
        "quantize_per_tensor_int8": [P, I, I64, P, P, P],
        "gemm_w8a8_requant": [P, P, P, P, P, I, P, I64, P, I64, I64, I64, P],
        "quantize_weight_per_channel_e4m3": [P, I64, I64, P, P, P],
        "gemm_e4m3_per_channel": [P, P, P, P, P, I, P, I, I64, I64, I64, P],
        "quantize_weight_block_asym_u8": [P, I64, I64, I64, P, P, P, P],
        "quantize_weight_int4_grouped": [P, I64, I64, I64, P, P, P],
    }
    for name, args in sig.items():
        getattr(L, name).argtypes = args
        getattr(L, name).restype = I
    L.ql_status_str.argtypes = [I]
    L.ql_status_str.restype = ctypes.c_char_p
    return L


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("quantize_per_row_int8", "quantize_weight_per_channel", "gemm_w8a8_per_channel",
              "gemm_w8a16", "gemm_w4a16_grouped", "gemm_w8a8_int32", "ql_status_str",
              "quantize_weight_block_asym_u8", "quantize_weight_int4_grouped",
              "gemm_w8a8_per_channel_act", "gemm_w4a16_grouped_act", "quantize_per_row_int8_asym",
              "weight_column_sums_i8", "gemm_w8a8_asym", "quantize_per_row_e4m3",
              "quantize_weight_per_channel_e4m3", "gemm_e4m3_per_channel",
              "quantize_per_tensor_int8", "gemm_w8a8_requant"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared():
        assert name in exported, name
        getattr(lib, name)


def test_no_undefined_library_symbols():
    """Every symbol the library references from itself is defined (a kernel whose launch stub
    the compiler did not emit would otherwise fail only when first called)."""
    if not os.path.exists(LIB):
        pytest.skip("libql.so not built")
    out = subprocess.run(["nm", "-C", "-D", "--undefined-only", LIB], capture_output=True,
                         text=True).stdout
    own = [l for l in out.splitlines() if "ql::" in l or "stub" in l]
    assert not own, own


def test_library_is_gfx950_only():
    """The embedded device code objects target gfx950 and nothing else."""
    if not os.path.exists(LIB):
        pytest.skip("libql.so not built")
    blob = open(LIB, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_status_strings(lib):
    for s in range(6):
        assert lib.ql_status_str(s)
    assert b"NULL" in lib.ql_status_str(NULL)


def test_quantize_per_row_validation(lib):
    f = lib.quantize_per_row_int8
    assert f(None, F16, 4, 64, A, A, None) == NULL
    assert f(A, F16, 4, 64, None, A, None) == NULL
    assert f(A, F16, 4, 64, A, None, None) == NULL
    assert f(A, 7, 4, 64, A, A, None) == DTYPE
    assert f(A, F16, -1, 64, A, A, None) == SHAPE
    assert f(A, F16, 4, 0, A, A, None) == SHAPE
    assert f(A, F16, 4, 24, A, A, None) == SHAPE
    assert f(MIS, F16, 4, 64, A, A, None) == ALIGN
    assert f(A, F16, 4, 64, MIS, A, None) == ALIGN
    assert f(A, F32, 4, 64, A, MIS, None) == ALIGN
    # an empty batch is a no-op, whatever the pointers
    assert f(None, F16, 0, 64, None, None, None) == OK


def test_quantize_weight_validation(lib):
    f = lib.quantize_weight_per_channel
    assert f(None, 64, 8, A, A, None) == NULL
    assert f(A, 63, 8, A, A, None) == SHAPE
    assert f(A, 64, -8, A, A, None) == SHAPE
    assert f(A, 64, 8, MIS, A, None) == ALIGN
    assert f(None, 64, 0, None, None, None) == OK


def test_gemm_w8a8_validation(lib):
    f = lib.gemm_w8a8_per_channel
    assert f(None, A, A, A, None, A, F16, 8, 8, 64, None) == NULL
    assert f(A, None, A, A, None, A, F16, 8, 8, 64, None) == NULL
    assert f(A, A, A, None, None, A, F16, 8, 8, 64, None) == NULL
    assert f(A, A, A, A, None, None, F16, 8, 8, 64, None) == NULL
    assert f(A, A, A, A, None, A, 3, 8, 8, 64, None) == DTYPE
    assert f(A, A, A, A, None, A, F16, 8, 8, 96, None) == SHAPE
    assert f(A, A, A, A, None, A, F16, 8, 8, 131072, None) == SHAPE
    assert f(A, A, A, A, None, A, F16, -1, 8, 64, None) == SHAPE
    assert f(A, A, A, A, None, A, F16, 8, 8, 0, None) == SHAPE
    assert f(A, A, MIS, A, None, A, F16, 8, 8, 64, None) == ALIGN
    assert f(A, A, A, A, MIS, A, F16, 8, 8, 64, None) == ALIGN
    assert f(None, None, None, None, None, None, F16, 0, 8, 64, None) == OK
    g = lib.gemm_w8a8_int32
    assert g(None, A, A, 8, 8, 64, None) == NULL
    assert g(A, A, A, 8, 8, 65, None) == SHAPE
    assert g(A, A, MIS, 8, 8, 64, None) == ALIGN
    assert g(None, None, None, 8, 0, 64, None) == OK


def test_gemm_w8a16_validation(lib):
    f = lib.gemm_w8a16
    assert f(None, A, A, None, 0, None, A, 1, 64, 128, None) == NULL
    assert f(A, A, None, None, 0, None, A, 1, 64, 128, None) == NULL
    assert f(A, A, A, None, 0, None, A, 1, 64, 100, None) == SHAPE
    assert f(A, A, A, A, 96, None, A, 1, 64, 192, None) == SHAPE     # group not a multiple of 64
    assert f(A, A, A, A, 128, None, A, 1, 64, 192, None) == SHAPE    # group does not divide K
    assert f(A, A, A, None, -64, None, A, 1, 64, 128, None) == SHAPE
    assert f(A, MIS, A, None, 0, None, A, 1, 64, 128, None) == ALIGN
    assert f(A, A, A, None, 0, None, MIS, 1, 64, 128, None) == ALIGN
    assert f(None, None, None, None, 0, None, None, 0, 64, 128, None) == OK


def test_gemm_w4a16_validation(lib):
    f = lib.gemm_w4a16_grouped
    assert f(None, A, A, 128, None, A, 32, 64, 256, None) == NULL
    assert f(A, A, None, 128, None, A, 32, 64, 256, None) == NULL
    assert f(A, A, A, 0, None, A, 32, 64, 256, None) == SHAPE
    assert f(A, A, A, 96, None, A, 32, 64, 384, None) == SHAPE
    assert f(A, A, A, 128, None, A, 32, 64, 320, None) == SHAPE
    assert f(A, MIS, A, 128, None, A, 32, 64, 256, None) == ALIGN
    assert f(A, A, MIS, 128, None, A, 32, 64, 256, None) == ALIGN
    assert f(None, None, None, 128, None, None, 32, 0, 256, None) == OK


def test_fused_activation_validation(lib):
    """The activation entry points validate like the plain ones, plus the activation code."""
    f = lib.gemm_w8a8_per_channel_act
    for act in (0, 1, 2):
        assert f(None, None, None, None, None, act, None, F16, 0, 8, 64, None) == OK
        assert f(A, A, A, A, None, act, None, F16, 8, 8, 64, None) == NULL
        assert f(A, A, A, A, None, act, A, F16, 8, 8, 96, None) == SHAPE
        assert f(A, A, MIS, A, None, act, A, F16, 8, 8, 64, None) == ALIGN
    assert f(A, A, A, A, None, 3, A, F16, 8, 8, 64, None) == DTYPE
    assert f(A, A, A, A, None, -1, A, F16, 8, 8, 64, None) == DTYPE
    assert f(A, A, A, A, None, 1, A, 3, 8, 8, 64, None) == DTYPE
    g = lib.gemm_w4a16_grouped_act
    for act in (0, 1, 2):
        assert g(None, None, None, 128, None, act, None, 32, 0, 256, None) == OK
        assert g(None, A, A, 128, None, act, A, 32, 64, 256, None) == NULL
        assert g(A, A, A, 96, None, act, A, 32, 64, 384, None) == SHAPE
        assert g(A, A, MIS, 128, None, act, A, 32, 64, 256, None) == ALIGN
    assert g(A, A, A, 128, None, 7, A, 32, 64, 256, None) == DTYPE


def test_asymmetric_validation(lib):
    f = lib.quantize_per_row_int8_asym
    assert f(A, F16, 0, 64, None, None, None, None) == OK
    assert f(A, 7, 4, 64, A, A, A, None) == DTYPE
    assert f(A, F16, 4, 40, A, A, A, None) == SHAPE
    assert f(A, F16, 4, 64, A, A, None, None) == NULL
    assert f(A, F16, 4, 64, A, A, MIS, None) == ALIGN
    g = lib.weight_column_sums_i8
    assert g(None, 64, 0, None, None) == OK
    assert g(A, 40, 8, A, None) == SHAPE
    assert g(None, 64, 8, A, None) == NULL
    assert g(MIS, 64, 8, A, None) == ALIGN
    h = lib.gemm_w8a8_asym
    assert h(None, None, None, None, None, None, None, 0, None, F16, 0, 8, 64, None) == OK
    assert h(A, A, None, A, A, A, None, 0, A, F16, 8, 8, 64, None) == NULL     # no zero points
    assert h(A, A, A, A, A, None, None, 0, A, F16, 8, 8, 64, None) == NULL     # no column sums
    assert h(A, A, A, A, A, A, None, 3, A, F16, 8, 8, 64, None) == DTYPE
    assert h(A, A, A, A, A, A, None, 1, A, 5, 8, 8, 64, None) == DTYPE
    assert h(A, A, A, A, A, A, None, 0, A, F16, 8, 8, 96, None) == SHAPE
    assert h(A, A, MIS, A, A, A, None, 0, A, F16, 8, 8, 64, None) == ALIGN
    assert h(A, A, A, A, A, MIS, None, 0, A, F16, 8, 8, 64, None) == ALIGN


def test_e4m3_validation(lib):
    f = lib.quantize_per_row_e4m3
    assert f(A, F16, 0, 64, None, None, None) == OK
    assert f(A, 7, 4, 64, A, A, None) == DTYPE
    assert f(A, F16, 4, 40, A, A, None) == SHAPE
    assert f(A, F16, 4, 64, None, A, None) == NULL
    assert f(MIS, F16, 4, 64, A, A, None) == ALIGN
    g = lib.quantize_weight_per_channel_e4m3
    assert g(None, 64, 0, None, None, None) == OK
    assert g(A, 40, 8, A, A, None) == SHAPE
    assert g(A, 64, 8, A, None, None) == NULL
    assert g(A, 64, 8, MIS, A, None) == ALIGN
    h = lib.gemm_e4m3_per_channel
    assert h(None, None, None, None, None, 0, None, F16, 8, 0, 64, None) == OK
    assert h(A, None, A, A, None, 0, A, F16, 8, 8, 64, None) == NULL
    assert h(A, A, A, A, None, 3, A, F16, 8, 8, 64, None) == DTYPE
    assert h(A, A, A, A, None, 0, A, 5, 8, 8, 64, None) == DTYPE
    assert h(A, A, A, A, None, 0, A, F16, 8, 8, 96, None) == SHAPE
    assert h(A, A, A, A, None, 0, A, F16, 8, 8, 131072, None) == SHAPE
    assert h(A, A, MIS, A, None, 0, A, F16, 8, 8, 64, None) == ALIGN
    assert h(A, A, A, A, MIS, 0, A, F16, 8, 8, 64, None) == ALIGN


def test_per_tensor_validation(lib):
    f = lib.quantize_per_tensor_int8
    assert f(None, F16, 0, None, None, None) == OK
    assert f(A, 7, 64, A, A, None) == DTYPE
    assert f(A, F16, 40, A, A, None) == SHAPE
    assert f(A, F16, -16, A, A, None) == SHAPE
    assert f(A, F16, 64, A, None, None) == NULL
    assert f(A, F16, 64, MIS, A, None) == ALIGN


def test_requant_validation(lib):
    f = lib.gemm_w8a8_requant
    assert f(None, None, None, None, None, 0, None, 1, None, 0, 8, 64, None) == OK
    assert f(A, A, A, A, None, 3, A, 1, A, 4, 8, 64, None) == DTYPE
    assert f(A, A, A, A, None, 0, A, 2, A, 4, 8, 64, None) == SHAPE      # neither 1 nor N
    assert f(A, A, A, A, None, 0, A, 0, A, 4, 8, 64, None) == SHAPE
    assert f(A, A, A, A, None, 0, A, 1, A, 4, 8, 96, None) == SHAPE
    assert f(A, A, A, A, None, 0, None, 1, A, 4, 8, 64, None) == NULL
    assert f(A, None, A, A, None, 0, A, 1, A, 4, 8, 64, None) == NULL
    assert f(A, A, A, A, None, 0, MIS, 1, A, 4, 8, 64, None) == ALIGN
    assert f(A, A, A, A, None, 0, A, 1, MIS, 4, 8, 64, None) == ALIGN


def test_producer_validation(lib):
    f = lib.quantize_weight_block_asym_u8
    assert f(None, 128, 8, 64, A, A, A, None) == NULL
    assert f(A, 128, 8, 48, A, A, A, None) == SHAPE
    assert f(A, 128, 8, 0, A, A, A, None) == SHAPE
    assert f(A, 128, 8, 64, MIS, A, A, None) == ALIGN
    g = lib.quantize_weight_int4_grouped
    assert g(None, 256, 8, 128, A, A, None) == NULL
    assert g(A, 256, 8, 96, A, A, None) == SHAPE
    assert g(A, 256, 8, 128, MIS, A, None) == ALIGN


PROBE_HEADER = os.path.join(ROOT, "include", "ql_probe.h")
PROBE_LIB = os.path.join(ROOT, "int8_quantized_linear_amd", "libqlprobe.so")


def test_probe_library_exports_its_header():
    """The benchmark's measurement probes (a library of their own, not the layer) export
    every function their header declares, and reject bad arguments without launching."""
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libqlprobe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = set(re.findall(r"^\s*int\s+([a-z_0-9]+)\s*\(", text, re.M))
    assert names == {"qlp_cu_count", "qlp_mfma_i8", "qlp_mfma_i8_data", "qlp_stream_read"}
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert names <= exported
    L = ctypes.CDLL(PROBE_LIB)
    L.qlp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.qlp_stream_read.restype = ctypes.c_int
    L.qlp_mfma_i8_data.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.qlp_mfma_i8_data.restype = ctypes.c_int
    # no GPU here: the device query fails first and nothing is launched
    assert L.qlp_stream_read(A, 16, A, None) == -1
    assert L.qlp_mfma_i8_data(1, A, 16, A, 16, A, None) == -1
