#!/usr/bin/env python3
"""Benchmark of the quantized linear layer's hot path on one MI355X (gfx950).

One step is one pass of every step of the path over one batch of synthetic input, with
all inputs resident in HBM:
  1. per-row int8 quantization of X [2048, 4096] fp16            (W8A8 prefill layer)
  2. W8A8 GEMM M=2048 K=4096 N=11008 + fused dequant/bias, fp16 out
  3. W8A16 decode GEMV M=1 K=4096 N=4096 (per-channel int8 weights)
  4. block-asymmetric W8A16 M=8 K=4096 N=4096 (uint8, blocks of 64)
  5. W4A16 M=32 K=4096 N=14336 (int4, groups of 128)
Weight quantization is offline (done once, untimed). The decode weights are replicated
in enough distinct buffers (over 512 MiB per workload) that each step streams its
weights from HBM rather than from the 256 MB Infinity Cache.

Printed: one JSON line. ``value`` is the W8A8 prefill layer's throughput in TOPS
(2*M*N*K integer ops over the average time of steps 1 + 2); the decode workloads'
GB/s are reported alongside. The timed region runs exactly K steps, issued in groups of
GROUP steps: within a group each kernel's GROUP launches go back to back, bracketed by
one pair of HIP events on the stream the kernels run on. A kernel's time is the sum of
its bracketed intervals over K. It includes the stream's launch-to-launch gap (about a
microsecond) but no event between two launches; short groups keep the GEMM's launches
from running long enough on their own to lower the chip's clock more than a pass of the
path does. Every input that streams from HBM rotates over more than 512 MiB of copies
(the decode weights and the quantizer's X), so no launch finds it in the Infinity Cache. The
GEMM, compute-bound, runs as a GEMM benchmark does, on the same W at every launch (45 MB, kept
by the 256 MB Infinity Cache); ``gemm_cold_weights`` gives it with W read from HBM as well.
The warm-up steps (200 by default) bring the chip out of its idle state first: after only 10,
every kernel of the timed region ran slower for its first several groups (the GEMM up to 15%).
``roofline`` is the W8A8 GEMM's (the dominant kernel); ``rooflines`` holds one entry per
hot-path kernel, each beside the rocprofv3 kernel-trace average of the committed profile
when that profile was taken on the current kernel sources.

After the timed region, measured ceilings (libqlprobe.so, not part of the layer) are
reported beside the published peaks: the int8 MFMA rate from registers alone, with
random and with constant operands (the chip's power limit sets its clock, and MFMA power
depends on the operand bits), and the rate one launch reads a buffer of each
memory-bound kernel's byte count from HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 per-channel GEMM TOPS at Llama-7B shapes; W8A16 decode GEMV GB/s"
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, 5.0 PFLOP/s
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
ROTATE_BYTES = 512 << 20
GROUP = 10                     # steps per group of back-to-back launches in the timed region


def _algorithmic_bytes():
    import workloads as wl
    w2, w4, w5, w3 = wl.W8A16_DECODE, wl.W8A16_BLOCK, wl.W4A16_GROUP, wl.W8A8_PREFILL
    return {
        # weights + scales (+ zero points) + X + Y
        "w8a16": w2.N * w2.K + 4 * w2.N + 2 * w2.M * w2.K + 2 * w2.M * w2.N,
        "w8a16_block": (w4.N * w4.K + 4 * w4.N * (w4.K // 64) + w4.N * (w4.K // 64)
                        + 2 * w4.M * w4.K + 2 * w4.M * w4.N),
        "w4a16": (w5.N * w5.K // 2 + 2 * w5.N * (w5.K // 128) + 2 * w5.M * w5.K
                  + 2 * w5.M * w5.N),
        # fp16 X in, int8 codes and fp32 scales out
        "quant": 2 * w3.M * w3.K + w3.M * w3.K + 4 * w3.M,
    }


def _kernel_hash():
    src = os.path.join(ROOT, "int8_quantized_linear_amd", "csrc", "gemm_w8a8.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def _library_hash():
    """Hash of every source of libql.so (sorted by name), to tie profiles to the code."""
    csrc = os.path.join(ROOT, "int8_quantized_linear_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")) and name != "probes.hip":
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "ql.h"), "rb").read())
    return h.hexdigest()[:16]


def _traffic_for_gemm():
    """HBM bytes per launch of the W8A8 GEMM from committed rocprofv3 counter runs, or None
    if absent or taken on a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "gemm_w8a8_m2048_k4096_n11008_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != _kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _profiled_kernel_times():
    """Per-kernel rocprofv3 kernel-trace averages (microseconds) of this benchmark's default
    command, from profiles/kernel_times.json, or {} when that file was written for other
    kernel sources (its hash covers every HIP source of the library)."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return {}
    if rec.get("library_source_sha256_16") != _library_hash():
        return {}
    return rec.get("avg_us", {})


def cpu_baseline(target_s: float):
    """The oracle timed on this host on a bounded sample of the W8A8 prefill layer: the first
    R rows of X through per-row quantization, the exact int32 GEMM against all of W, and the
    epilogue. R is chosen so that one run takes about target_s / 3 seconds; the reported
    time is the median of three runs."""
    import numpy as np

    import oracle
    import workloads as wl

    w = wl.W8A8_PREFILL
    inp = wl.draw(w)
    wq, ws = oracle.quant_weight_per_channel(inp.w_nk)   # offline, untimed

    def run(r):
        t0 = time.perf_counter()
        res = oracle.linear_w8a8(inp.x[:r], wq, ws, inp.bias)
        _ = res["y32"].astype(np.float16)
        return time.perf_counter() - t0

    # rows are spread over the oracle's OpenMP threads: calibrate on one row per thread
    nt = max(1, min(64, oracle.num_threads()))
    per_row = run(nt) / nt
    rows = int(max(nt, min(w.M, nt * round(target_s / 3 / per_row / nt))))
    times = sorted(run(rows) for _ in range(3))
    dt = times[1]
    ops = 2.0 * rows * w.N * w.K
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "rows 0..%d of X [2048,4096] through the W8A8 layer (per-row quantize, exact "
                      "int32 GEMM with W [4096,11008], fp32 epilogue, fp16 output): median of 3 runs "
                      "of %.2f, %.2f, %.2f s" % (rows - 1, *times),
            "seconds": dt, "host": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "single_thread": _cpu_single_thread(target_s / 6)}


_ONE_THREAD = r"""
import sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle, workloads as wl
w = wl.W8A8_PREFILL
inp = wl.draw(w)
wq, ws = oracle.quant_weight_per_channel(inp.w_nk)
t0 = time.perf_counter(); oracle.linear_w8a8(inp.x[:1], wq, ws, inp.bias); per_row = time.perf_counter() - t0
rows = int(max(1, min(w.M, round(float(sys.argv[2]) / per_row))))
ts = []
for _ in range(3):
    t0 = time.perf_counter(); r = oracle.linear_w8a8(inp.x[:rows], wq, ws, inp.bias); ts.append(time.perf_counter() - t0)
print(rows, sorted(ts)[1], oracle.num_threads())
"""


def _cpu_single_thread(target_s: float):
    """The same oracle sample on one thread (median of three runs), in a child process
    started with OMP_NUM_THREADS=1 (the oracle reads it when its library loads)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _ONE_THREAD, ROOT, str(target_s)], env=env,
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1:] or ["failed"]}
    rows, dt, threads = r.stdout.split()
    rows, dt = int(rows), float(dt)
    w = 2.0 * rows * 11008 * 4096
    return {"value": w / dt / 1e12, "unit": "TOPS", "cores": int(threads), "rows": rows, "seconds": dt}


def _cycle(launches):
    """A zero-argument callable that launches the next of `launches` at each call."""
    state = [0]

    def f():
        launches[state[0] % len(launches)]()
        state[0] += 1
    return f


def fused_activation_timings(ql, n, gemm, dec5, make_gemm, make_dec, ops, w4_bytes, gemm_name,
                             dec_name, progress):
    """The epilogue with a fused activation (GELU, SiLU) against the plain epilogue: the
    W8A8 GEMM at the prefill shape and W4A16 at the decode shape. Plain and fused bursts
    alternate so that both run at the same clock; the decode weights rotate as in the
    step loop."""
    progress("fused activations: %d bursts each" % n)
    gelu, silu = ql.ACTIVATIONS["gelu"], ql.ACTIVATIONS["silu"]
    us = _alternate(n, {"w8a8_plain": gemm, "w8a8_gelu": make_gemm(gelu), "w8a8_silu": make_gemm(silu),
                        "w4a16_plain": _cycle(dec5), "w4a16_gelu": _cycle(make_dec(gelu))})
    return {
        gemm_name: {"plain_us": us["w8a8_plain"], "gelu_us": us["w8a8_gelu"], "silu_us": us["w8a8_silu"],
                    "gelu_TOPS": ops / (us["w8a8_gelu"] * 1e-6) / 1e12,
                    "gelu_overhead": us["w8a8_gelu"] / us["w8a8_plain"] - 1,
                    "silu_overhead": us["w8a8_silu"] / us["w8a8_plain"] - 1},
        dec_name: {"plain_us": us["w4a16_plain"], "gelu_us": us["w4a16_gelu"],
                   "gelu_GB_per_s": w4_bytes / (us["w4a16_gelu"] * 1e-6) / 1e9,
                   "gelu_overhead": us["w4a16_gelu"] / us["w4a16_plain"] - 1},
        "note": "bursts of plain and fused launches alternate; event-timed per burst",
    }


BURST = 10


def _alternate(n, runs):
    """Mean microseconds per launch of each zero-argument callable in runs: one warm-up
    burst each, then n rounds in which each callable runs a burst of BURST back-to-back
    launches bracketed by one event pair, the callables alternating burst by burst."""
    import torch
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
          for k in runs}
    for f in runs.values():
        for _ in range(BURST):
            f()
    torch.cuda.synchronize()
    for i in range(n):
        for k, f in runs.items():
            ev[k][i][0].record()
            for _ in range(BURST):
                f()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    return {k: 1e3 * sum(a.elapsed_time(b) for a, b in v) / (n * BURST) for k, v in ev.items()}


def small_layer_graph_us(ql, x, xq, xs, wq, ws, b, y, w, layers=20, replays=20):
    """Microseconds per layer (per-row quantizer + GEMM) of a small layer whose launches are
    captured in a HIP graph (`layers` layers per graph) and replayed: the device-side latency,
    without the host's launch cost that bursts of launches from Python include."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        ql.prepare("quantize_per_row_int8", x, 0, w.M, w.K, xq, xs)()
        ql.prepare("gemm_w8a8_per_channel", xq, xs, wq, ws, b, y, 0, w.M, w.N, w.K)()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        # prepared inside the capture, so that they launch on the capturing stream
        q = ql.prepare("quantize_per_row_int8", x, 0, w.M, w.K, xq, xs)
        m = ql.prepare("gemm_w8a8_per_channel", xq, xs, wq, ws, b, y, 0, w.M, w.N, w.K)
        for _ in range(layers):
            q()
            m()
    g.replay()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(e) / (replays * layers)


def asym_timings(n, runs, ops, quant_bytes, name, progress):
    """The layer with asymmetric per-row activations (quantizer with a float zero point, GEMM
    with the zero-point correction in the epilogue) against the symmetric one at the same
    shape: each launch event-timed, the four alternating."""
    progress("asymmetric activations: %d launches each" % n)
    us = _alternate(n, runs)
    layer = us["quant_asym"] + us["gemm_asym"]
    return {name: {"quant_us": us["quant_asym"], "gemm_us": us["gemm_asym"],
                   "quant_GB_per_s": quant_bytes / (us["quant_asym"] * 1e-6) / 1e9 + 0.0,
                   "layer_TOPS": ops / (layer * 1e-6) / 1e12,
                   "symmetric_quant_us": us["quant_symmetric"], "symmetric_gemm_us": us["gemm_symmetric"],
                   "gemm_overhead": us["gemm_asym"] / us["gemm_symmetric"] - 1},
            "note": "quantizer bytes: fp16 X in, int8 codes out, scale and zero point per row"}


def fp8_timings(n, runs, ops, quant_bytes, name, progress):
    """The fp8 (E4M3) layer at the prefill shape (per-row fp8 quantizer, fp8 GEMM with fp32
    accumulation and the same epilogue) against the int8 layer, launches alternating."""
    progress("fp8 layer: %d launches each" % n)
    us = _alternate(n, runs)
    tf = ops / (us["gemm_e4m3"] * 1e-6) / 1e12
    return {name: {"quant_us": us["quant_e4m3"], "gemm_us": us["gemm_e4m3"],
                   "quant_GB_per_s": quant_bytes / (us["quant_e4m3"] * 1e-6) / 1e9,
                   "gemm_TFLOPS": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
                   "layer_TFLOPS": ops / ((us["quant_e4m3"] + us["gemm_e4m3"]) * 1e-6) / 1e12,
                   "int8_quant_us": us["quant_int8"], "int8_gemm_us": us["gemm_int8"],
                   "gemm_time_vs_int8": us["gemm_e4m3"] / us["gemm_int8"]},
            "note": "2*M*N*K flops per GEMM launch against the dense fp8 MFMA peak (5.0 PFLOP/s)"}


def requant_timings(n, runs, ops, name, progress):
    """The W8A8 GEMM with its output re-quantized to int8 in the epilogue (static scales)
    against the plain fp16-output GEMM, and against the unfused pair that a per-row dynamic
    re-quantization needs (fp16 GEMM, then the per-row quantizer over Y); alternating."""
    progress("int8 output: %d launches each" % n)
    us = _alternate(n, runs)
    return {name: {"requant_gemm_us": us["gemm_requant"], "plain_fp16_gemm_us": us["gemm_fp16"],
                   "requant_TOPS": ops / (us["gemm_requant"] * 1e-6) / 1e12,
                   "requant_vs_plain": us["gemm_requant"] / us["gemm_fp16"],
                   "unfused_gemm_plus_row_quant_us": us["gemm_fp16"] + us["quant_y_rows"],
                   "row_quant_of_y_us": us["quant_y_rows"]},
            "note": "int8 Y halves the output bytes (45 MB of fp16 to 22.5 MB)"}


def producer_timings(n, runs, nbytes, progress):
    """The quantizers that feed the path, each event-timed with launches alternating: the
    per-tensor quantizer on the prefill activations (four launches per call: clear, absmax,
    codes, scale) and the offline weight producers at their workloads' shapes. GB/s counts
    each kernel's algorithmic bytes (inputs read once, outputs written once)."""
    progress("producers: %d launches each" % n)
    us = _alternate(n, runs)
    return {k: {"us": us[k], "GB_per_s": nbytes[k] / (us[k] * 1e-6) / 1e9} for k in runs}


def measured_ceilings(dev, byte_counts, progress, layer_codes=None):
    """Ceilings measured with libqlprobe.so: int8 MFMA TOPS from registers (random and
    constant operands, and the layer's own W and X codes when `layer_codes` = (wq, xq) is
    given) and the GB/s of one cold streaming read of each byte count."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "int8_quantized_linear_amd", "libqlprobe.so")
    if not os.path.exists(path):
        raise RuntimeError("libqlprobe.so is not built at %s" % path)
    P = ctypes.CDLL(path)
    P.qlp_cu_count.restype = ctypes.c_int
    P.qlp_mfma_i8.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.qlp_mfma_i8.restype = ctypes.c_int
    P.qlp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    P.qlp_stream_read.restype = ctypes.c_int
    P.qlp_mfma_i8_data.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    P.qlp_mfma_i8_data.restype = ctypes.c_int
    cus = P.qlp_cu_count()
    if cus <= 0:
        raise RuntimeError("qlp_cu_count failed")
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.empty(cus * 512, dtype=torch.int32, device=dev)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with %d" % (what, rc))

    def timed(fn, reps):
        # one event pair around reps back-to-back launches, as for the layer's kernels
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3   # seconds per launch

    progress("measured ceilings")
    out = {"mfma_i8_TOPS": {}, "stream_read_GB_per_s": {}}
    iters = 2000
    ops = float(cus) * 4 * iters * 16 * 65536
    for name, rnd in (("random_operands", 1), ("constant_operands", 0)):
        check(P.qlp_mfma_i8(100, rnd, ctypes.c_void_p(sink.data_ptr()), sh), "qlp_mfma_i8")
        dt = timed(lambda i: check(P.qlp_mfma_i8(iters, rnd, ctypes.c_void_p(sink.data_ptr()), sh),
                                   "qlp_mfma_i8"), 5)
        out["mfma_i8_TOPS"][name] = ops / dt / 1e12
    if layer_codes is not None:
        wq, xq = layer_codes
        wb, xb = wq.numel() // 16 * 16, xq.numel() // 16 * 16

        def data_launch(n):
            check(P.qlp_mfma_i8_data(n, ctypes.c_void_p(wq.data_ptr()), wb, ctypes.c_void_p(xq.data_ptr()), xb,
                                     ctypes.c_void_p(sink.data_ptr()), sh), "qlp_mfma_i8_data")
        data_launch(100)
        dt = timed(lambda i: data_launch(iters), 5)
        out["mfma_i8_TOPS"]["layer_operands"] = ops / dt / 1e12
    for name, nbytes in byte_counts.items():
        nb = (nbytes + 15) // 16 * 16
        nbuf = max(2, math.ceil(ROTATE_BYTES / nb))
        bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        torch.cuda.synchronize()
        reps = 2 * nbuf
        dt = timed(lambda i: check(P.qlp_stream_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nb,
                                                     ctypes.c_void_p(sink.data_ptr()), sh),
                                   "qlp_stream_read"), reps)
        out["stream_read_GB_per_s"][name] = nb / dt / 1e9
        del bufs
    out["note"] = ("MFMA: %d workgroups x 4 waves issuing v_mfma_i32_32x32x32_i8 from registers (layer_operands: "
                   "fragments loaded once from the W8A8 layer's own W and X codes, W first as in the GEMM); "
                   "stream read: launches reading a cold buffer of each kernel's algorithmic "
                   "byte count (buffers rotated over more than 512 MiB), timed as a back-to-back burst" % cus)
    return out


def read_sweep(dev, progress):
    """Cold streaming reads of 16 MiB to 1 GiB with the probe of libqlprobe.so (buffers rotated
    over at least 1.5 GiB, two for the largest), each size timed as a burst of back-to-back
    launches between two events; under rocprofv3 --kernel-trace the same command gives each
    launch's duration. Returns {MiB: {"us": per launch, "GB_per_s": ...}}."""
    import ctypes

    import torch

    P = ctypes.CDLL(os.path.join(ROOT, "int8_quantized_linear_amd", "libqlprobe.so"))
    P.qlp_cu_count.restype = ctypes.c_int
    P.qlp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    P.qlp_stream_read.restype = ctypes.c_int
    cus = P.qlp_cu_count()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.empty(cus * 512, dtype=torch.int32, device=dev)
    out = {}
    for mib in (16, 32, 64, 128, 256, 512, 1024):
        nb = mib << 20
        nbuf = 2 if mib >= 1024 else max(2, (1536 << 20) // nb)
        bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        reps = max(8, min(2 * nbuf, 96))
        for i in range(nbuf):
            P.qlp_stream_read(ctypes.c_void_p(bufs[i].data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()), sh)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            rc = P.qlp_stream_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()), sh)
            if rc != 0:
                raise RuntimeError("qlp_stream_read failed with %d" % rc)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        out[mib] = {"us": us, "GB_per_s": nb / us / 1e3, "launches": reps, "buffers": nbuf}
        progress("read %d MiB: %.2f us per launch (%.0f GB/s)" % (mib, us, nb / us / 1e3))
        del bufs
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The chip ramps up from idle: with 10 warm-up steps the GEMM's groups of the timed region ran
    # 91.6, 99.1, 100.3, 96.2, ..., 85.6 us; after 100 they hold at 85-86 us from the first group.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=18.0)
    ap.add_argument("--act-steps", type=int, default=20,
                    help="launches of each fused-activation variant timed after the step loop (0: skip)")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false",
                    help="skip the measured ceilings (MFMA-only and streaming-read probes)")
    ap.add_argument("--read-sweep", action="store_true",
                    help="only measure cold streaming reads of 16 MiB .. 1 GiB with the probe and print them")
    ap.add_argument("--calib-copy-mib", type=int, default=256,
                    help="size of the plain device copy run once before the timed region "
                         "(reference point for hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_quantized_linear_amd as ql
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.read_sweep:
        res = read_sweep(dev, lambda m: print("[bench] " + m, file=sys.stderr, flush=True))
        print(json.dumps({"read_sweep_MiB": res, "device": torch.cuda.get_device_name(0)}), flush=True)
        return

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def progress(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- inputs
    progress("drawing inputs")
    w3 = wl.W8A8_PREFILL
    i3 = wl.draw(w3)
    wq3, ws3 = ql.quantize_weight_per_channel(up(i3.w_nk))
    x3, b3 = up(i3.x), up(i3.bias)
    xq3 = torch.empty((w3.M, w3.K), dtype=torch.int8, device=dev)
    xs3 = torch.empty((w3.M,), dtype=torch.float32, device=dev)
    y3 = torch.empty((w3.M, w3.N), dtype=torch.float16, device=dev)
    if args.act_steps > 0:
        w3f = up(i3.w_nk)
        wq8, ws8 = ql.quantize_weight_per_channel_e4m3(w3f)
    del i3

    def rotations(nbytes):
        return max(2, math.ceil(ROTATE_BYTES / nbytes))

    ab = _algorithmic_bytes()
    w2 = wl.W8A16_DECODE
    i2 = wl.draw(w2)
    q2, s2 = ql.quantize_weight_per_channel(up(i2.w_nk))
    r2 = rotations(ab["w8a16"])
    set2 = [(q2.clone(), s2.clone()) for _ in range(r2)]
    x2 = up(i2.x)
    y2 = torch.empty((w2.M, w2.N), dtype=torch.float16, device=dev)

    w4 = wl.W8A16_BLOCK
    i4 = wl.draw(w4)
    q4, s4, z4 = ql.quantize_weight_block_asym_u8(up(i4.w_nk), 64)
    r4 = rotations(ab["w8a16_block"])
    set4 = [(q4.clone(), s4.clone(), z4.clone()) for _ in range(r4)]
    x4 = up(i4.x)
    y4 = torch.empty((w4.M, w4.N), dtype=torch.float16, device=dev)

    w5 = wl.W4A16_GROUP
    i5 = wl.draw(w5)
    p5, s5 = ql.quantize_weight_int4_grouped(up(i5.w_nk), 128)
    r5 = rotations(ab["w4a16"])
    set5 = [(p5.clone(), s5.clone()) for _ in range(r5)]
    x5 = up(i5.x)
    y5 = torch.empty((w5.M, w5.N), dtype=torch.float16, device=dev)
    del i2, i4, i5
    torch.cuda.synchronize()

    w1 = wl.W8A8_SMALL
    i1 = wl.draw(w1)
    wq1, ws1 = ql.quantize_weight_per_channel(up(i1.w_nk))
    x1, b1 = up(i1.x), up(i1.bias)
    xq1 = torch.empty((w1.M, w1.K), dtype=torch.int8, device=dev)
    xs1 = torch.empty((w1.M,), dtype=torch.float32, device=dev)
    y1 = torch.empty((w1.M, w1.N), dtype=torch.float32, device=dev)
    del i1

    # ------------------------------------------------- prepared launches
    F16 = 1
    rq = rotations(2 * w3.M * w3.K)
    xsets3 = [x3.clone() for _ in range(rq)]
    quants = [ql.prepare("quantize_per_row_int8", xc, F16, w3.M, w3.K, xq3, xs3) for xc in xsets3]
    gemm = ql.prepare("gemm_w8a8_per_channel", xq3, xs3, wq3, ws3, b3, y3, F16, w3.M, w3.N, w3.K)
    dec2 = [ql.prepare("gemm_w8a16", x2, q, s, None, 0, None, y2, w2.M, w2.N, w2.K) for q, s in set2]
    dec4 = [ql.prepare("gemm_w8a16", x4, q, s, z, 64, None, y4, w4.M, w4.N, w4.K) for q, s, z in set4]
    dec5 = [ql.prepare("gemm_w4a16_grouped", x5, p, s, 128, None, y5, w5.M, w5.N, w5.K) for p, s in set5]

    # the kernels of one step, in path order (decode weight sets rotate by step)
    burst = {"quant": lambda i: quants[i % rq](), "gemm": lambda i: gemm(), "w8a16": lambda i: dec2[i % r2](),
             "w8a16_block": lambda i: dec4[i % r4](), "w4a16": lambda i: dec5[i % r5]()}

    # Plain device copy of known size (reference for hardware byte counters), untimed.
    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    progress("warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        for f in burst.values():
            f(i)
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    names = list(burst)
    # Steps in groups of GROUP: within a group, each kernel's launches for the group's steps go
    # back to back between two events on the launch stream
    intervals = {n: [] for n in names}
    progress("timing %d steps" % K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g0 in range(0, K, GROUP):
        steps = range(args.warmup + g0, args.warmup + min(K, g0 + GROUP))
        for n in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in steps:
                burst[n](i)
            b.record(stream)
            intervals[n].append((a, b))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    avg_ms = {n: sum(a.elapsed_time(b) for a, b in intervals[n]) / K for n in names}

    ops = 2.0 * w3.M * w3.N * w3.K
    layer_s = (avg_ms["quant"] + avg_ms["gemm"]) * 1e-3
    gemm_s = avg_ms["gemm"] * 1e-3
    value = ops / layer_s / 1e12
    gemm_tops = ops / gemm_s / 1e12

    def gbs(name):
        return ab[name] / (avg_ms[name] * 1e-3) / 1e9

    prof = _profiled_kernel_times()
    decode = {}
    for name, w, rot in (("w8a16", w2, r2), ("w8a16_block", w4, r4), ("w4a16", w5, r5)):
        decode[name] = {"workload": w.name, "us": avg_ms[name] * 1e3, "GB_per_s": gbs(name),
                        "frac_hbm_peak": gbs(name) / PEAK_HBM_GBS, "bytes": ab[name],
                        "weight_sets_rotated": rot}
    rooflines = {}
    for name, kern in (("quant", "quantize_per_row_int8 " + w3.name), ("w8a16", "gemm_w8a16 " + w2.name),
                       ("w8a16_block", "gemm_w8a16 " + w4.name), ("w4a16", "gemm_w4a16_grouped " + w5.name)):
        r = {"bound": "hbm", "kernel": kern, "achieved": gbs(name), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": gbs(name) / PEAK_HBM_GBS, "avg_us": avg_ms[name] * 1e3, "bytes_per_launch": ab[name]}
        if name in prof:
            r["rocprof_avg_us"] = prof[name]
            r["frac_by_rocprof_avg"] = ab[name] / (prof[name] * 1e-6) / 1e9 / PEAK_HBM_GBS
        rooflines[name] = r
    roof = {"bound": "mfma", "kernel": "gemm_w8a8_per_channel " + w3.name, "achieved": gemm_tops,
            "peak": PEAK_INT8_TOPS, "unit": "TOPS", "frac": gemm_tops / PEAK_INT8_TOPS,
            "traffic": _traffic_for_gemm(), "avg_us": avg_ms["gemm"] * 1e3, "ops_per_launch": ops,
            "note": "int8 operations (2*M*N*K per launch) over the kernel's average time in the timed "
                    "steps, against the dense int8 MFMA peak (5.0 POP/s)"}
    if "gemm" in prof:
        roof["rocprof_avg_us"] = prof["gemm"]
        roof["frac_by_rocprof_avg"] = ops / (prof["gemm"] * 1e-6) / 1e12 / PEAK_INT8_TOPS
    rooflines["gemm"] = roof
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w3.name, "M": w3.M, "K": w3.K, "N": w3.N, "x": "fp16", "y": "fp16",
                   "bias": True, "value_covers": "per-row quantization + W8A8 GEMM",
                   "decode_workloads": [w2.name, w4.name, w5.name]},
        "roofline": roof,
        "rooflines": rooflines,
        "w8a16_decode_GB_per_s": decode["w8a16"]["GB_per_s"],
        "quantizer": {"us": avg_ms["quant"] * 1e3, "GB_per_s": gbs("quant"),
                      "frac_hbm_peak": gbs("quant") / PEAK_HBM_GBS},
        "decode": decode,
        "timing": "steps in groups of %d; within a group each kernel's launches run back to back between "
                  "two HIP events on the launch stream (includes the launch gap)" % GROUP,
        "gemm_us_by_group": [round(a.elapsed_time(b) * 1e3 / (min(K, g0 + GROUP) - g0), 2)
                             for g0, (a, b) in zip(range(0, K, GROUP), intervals["gemm"])],
        "device": torch.cuda.get_device_name(0),
    }
    if args.act_steps > 0:
        out["fused_activation"] = fused_activation_timings(
            ql, args.act_steps, gemm, dec5,
            lambda code: ql.prepare("gemm_w8a8_per_channel_act", xq3, xs3, wq3, ws3, b3, code, y3, F16,
                                    w3.M, w3.N, w3.K),
            lambda code: [ql.prepare("gemm_w4a16_grouped_act", x5, p, s, 128, None, code, y5, w5.M, w5.N,
                                     w5.K) for p, s in set5],
            ops, ab["w4a16"], w3.name, w5.name, progress)
    if args.act_steps > 0:
        # The decode kernels with one weight set launched over and over (its bytes stay in the
        # 256 MB Infinity Cache) against the rotated cold sets, bursts alternating: how much of a
        # launch the HBM accounts for, and how much the kernel's own on-chip work does.
        progress("decode with warm weights: %d bursts each" % args.act_steps)
        dsets = {"w8a16": dec2, "w8a16_block": dec4, "w4a16": dec5}
        runs = {}
        for name, decs in dsets.items():
            runs[name + "_cold"] = _cycle(decs)
            runs[name + "_warm"] = decs[0]
        us = _alternate(args.act_steps, runs)
        out["decode_warm_weights"] = {
            name: {"cold_us": us[name + "_cold"], "warm_us": us[name + "_warm"],
                   "warm_GB_per_s": ab[name] / (us[name + "_warm"] * 1e-6) / 1e9}
            for name in dsets}
        out["decode_warm_weights"]["note"] = (
            "bursts alternate between rotated weight sets (read from HBM) and one set launched "
            "repeatedly (served from the Infinity Cache); event-timed per burst")
    if args.act_steps > 0:
        # The timed step's GEMM, like a GEMM benchmark, launches on the same W each time (45 MB,
        # which the 256 MB Infinity Cache keeps between launches); here it also runs over copies of
        # W rotated through more than 512 MiB, so that every launch reads W from HBM, bursts
        # alternating with the resident W.
        progress("W8A8 GEMM with cold weights: %d bursts each" % args.act_steps)
        rw = rotations(w3.N * w3.K)
        wsets3 = [wq3.clone() for _ in range(rw)]
        gemms_cold = [ql.prepare("gemm_w8a8_per_channel", xq3, xs3, wq_, ws3, b3, y3, F16, w3.M, w3.N, w3.K)
                      for wq_ in wsets3]
        usg = _alternate(args.act_steps, {"resident": gemm, "cold": _cycle(gemms_cold)})
        out["gemm_cold_weights"] = {
            w3.name: {"resident_us": usg["resident"], "cold_us": usg["cold"], "weight_sets_rotated": rw,
                      "cold_TOPS": ops / (usg["cold"] * 1e-6) / 1e12,
                      "cold_frac_int8_peak": ops / (usg["cold"] * 1e-6) / 1e12 / PEAK_INT8_TOPS},
            "note": "bursts alternate between the timed step's W (resident) and copies of W rotated over "
                    "more than 512 MiB (read from HBM at every launch); event-timed per burst"}
        del wsets3, gemms_cold
    if args.act_steps > 0:
        xz3 = torch.empty((w3.M,), dtype=torch.float32, device=dev)
        cs3 = ql.weight_column_sums_i8(wq3)
        out["asymmetric_activations"] = asym_timings(
            args.act_steps, {
                "quant_symmetric": _cycle(quants), "gemm_symmetric": gemm,
                "quant_asym": _cycle([ql.prepare("quantize_per_row_int8_asym", xc, F16, w3.M, w3.K, xq3, xs3, xz3)
                                      for xc in xsets3]),
                "gemm_asym": ql.prepare("gemm_w8a8_asym", xq3, xs3, xz3, wq3, ws3, cs3, b3, 0, y3, F16,
                                        w3.M, w3.N, w3.K)},
            ops, ab["quant"] + 4 * w3.M, w3.name, progress)
    if args.act_steps > 0:
        xq8 = torch.empty((w3.M, w3.K), dtype=torch.float8_e4m3fn, device=dev)
        xs8 = torch.empty((w3.M,), dtype=torch.float32, device=dev)
        out["fp8"] = fp8_timings(
            args.act_steps, {
                "quant_int8": _cycle(quants), "gemm_int8": gemm,
                "quant_e4m3": _cycle([ql.prepare("quantize_per_row_e4m3", xc, F16, w3.M, w3.K, xq8, xs8)
                                      for xc in xsets3]),
                "gemm_e4m3": ql.prepare("gemm_e4m3_per_channel", xq8, xs8, wq8, ws8, b3, 0, y3, F16,
                                        w3.M, w3.N, w3.K)},
            ops, ab["quant"], w3.name, progress)
    if args.act_steps > 0:
        progress("small layer latency: %d launches each" % args.act_steps)
        us1 = _alternate(args.act_steps, {
            "quant": ql.prepare("quantize_per_row_int8", x1, 0, w1.M, w1.K, xq1, xs1),
            "gemm": ql.prepare("gemm_w8a8_per_channel", xq1, xs1, wq1, ws1, b1, y1, 0, w1.M, w1.N, w1.K)})
        out["small_layer"] = {"workload": w1.name, "quant_us": us1["quant"], "gemm_us": us1["gemm"],
                              "layer_us": us1["quant"] + us1["gemm"],
                              "graph_layer_us": small_layer_graph_us(ql, x1, xq1, xs1, wq1, ws1, b1, y1, w1),
                              "note": "latency-bound: 16 quantizer workgroups (one per row), then the few-row GEMM kernel "
                                      "(16 workgroups of 16 columns); bursts event-timed (host launch rate included); "
                                      "graph_layer_us: the two launches replayed from a HIP graph, no host launch cost"}
    if args.act_steps > 0:
        # W8A8 with few rows (decode-time batches) at the 4096 x 4096 decode shape, weights
        # rotated like the decode kernels' so every launch reads W from HBM
        nk = w2.N * w2.K
        rot = max(2, math.ceil(ROTATE_BYTES / nk))
        wsets = [torch.randint(-127, 128, (w2.N, w2.K), dtype=torch.int8, device=dev) for _ in range(rot)]
        wsc = torch.rand(w2.N, device=dev) * 0.01
        few = {}
        for m in (1, 16):
            xqm = torch.randint(-127, 128, (m, w2.K), dtype=torch.int8, device=dev)
            xsm = torch.rand(m, device=dev) * 0.01
            ym = torch.empty((m, w2.N), dtype=torch.float16, device=dev)
            launches = [ql.prepare("gemm_w8a8_per_channel", xqm, xsm, wq_, wsc, None, ym, F16, m, w2.N, w2.K)
                        for wq_ in wsets]
            us = _alternate(args.act_steps, {"run": _cycle(launches)})["run"]
            few["m%d" % m] = {"us": us, "GB_per_s": nk / (us * 1e-6) / 1e9}
        out["w8a8_few_rows"] = {"shape": "M x K4096 x N4096, fp16 out", "weight_sets_rotated": rot, **few,
                                "note": "M <= 8, or M <= 128 with M*N <= 256K and N <= 12288, runs on the few-row kernel; GB/s counts W's bytes; timed after "
                                        "the GEMM runs above, whose power draw can leave the clock lower"}
        del wsets
    if args.act_steps > 0:
        s_out = torch.full((w3.N,), 0.02, dtype=torch.float32, device=dev)
        yq3 = torch.empty((w3.M, w3.N), dtype=torch.int8, device=dev)
        yqs = torch.empty((w3.M,), dtype=torch.float32, device=dev)
        out["int8_output"] = requant_timings(args.act_steps, {
            "gemm_fp16": gemm,
            "gemm_requant": ql.prepare("gemm_w8a8_requant", xq3, xs3, wq3, ws3, b3, 0, s_out, w3.N, yq3,
                                       w3.M, w3.N, w3.K),
            "quant_y_rows": ql.prepare("quantize_per_row_int8", y3, F16, w3.M, w3.N, yq3, yqs),
        }, ops, w3.name, progress)
        w4f = up(wl.draw(w4, x_rows=slice(0, 1)).w_nk)
        w5f = up(wl.draw(w5, x_rows=slice(0, 1)).w_nk)
        xqt = torch.empty((w3.M, w3.K), dtype=torch.int8, device=dev)
        xst = torch.empty((1,), dtype=torch.float32, device=dev)
        pq3 = torch.empty_like(wq3)
        ps3 = torch.empty_like(ws3)
        pq8 = torch.empty_like(wq8)
        pq4 = torch.empty((w4.N, w4.K), dtype=torch.uint8, device=dev)
        ps4 = torch.empty((w4.N, w4.K // 64), dtype=torch.float32, device=dev)
        pz4 = torch.empty((w4.N, w4.K // 64), dtype=torch.uint8, device=dev)
        pp5 = torch.empty((w5.N, w5.K // 8), dtype=torch.int32, device=dev)
        ps5 = torch.empty((w5.N, w5.K // 128), dtype=torch.float16, device=dev)
        mk3, n3, n4, n5 = w3.M * w3.K, w3.N * w3.K, w4.N * w4.K, w5.N * w5.K
        out["producers"] = producer_timings(args.act_steps, {
            "per_tensor_int8_x_" + w3.name: ql.prepare("quantize_per_tensor_int8", x3, F16, mk3, xqt, xst),
            "per_channel_int8_w_" + w3.name: ql.prepare("quantize_weight_per_channel", w3f, w3.K, w3.N, pq3, ps3),
            "per_channel_e4m3_w_" + w3.name: ql.prepare("quantize_weight_per_channel_e4m3", w3f, w3.K, w3.N, pq8, ps3),
            "block64_asym_u8_w_" + w4.name: ql.prepare("quantize_weight_block_asym_u8", w4f, w4.K, w4.N, 64, pq4, ps4, pz4),
            "int4_g128_w_" + w5.name: ql.prepare("quantize_weight_int4_grouped", w5f, w5.K, w5.N, 128, pp5, ps5),
        }, {
            "per_tensor_int8_x_" + w3.name: 3 * mk3 + 4,
            "per_channel_int8_w_" + w3.name: 5 * n3 + 4 * w3.N,
            "per_channel_e4m3_w_" + w3.name: 5 * n3 + 4 * w3.N,
            "block64_asym_u8_w_" + w4.name: 5 * n4 + 5 * (n4 // 64),
            "int4_g128_w_" + w5.name: 4 * n5 + n5 // 2 + 2 * (n5 // 128),
        }, progress)
        del w3f, w4f, w5f
    if args.ceilings:
        del set2, set4, set5, dec2, dec4, dec5
        ceil = measured_ceilings(dev, {"quant": ab["quant"], "w8a16": ab["w8a16"],
                                       "w8a16_block": ab["w8a16_block"], "w4a16": ab["w4a16"]}, progress,
                                 layer_codes=(wq3, xq3))
        out["ceilings"] = ceil
        mc = ceil["mfma_i8_TOPS"]["random_operands"]
        out["roofline"]["measured_ceiling"] = mc
        out["roofline"]["frac_of_measured_ceiling"] = gemm_tops / mc
        out["roofline"]["frac_of_layer_operand_ceiling"] = gemm_tops / ceil["mfma_i8_TOPS"]["layer_operands"]
        rd = ceil["stream_read_GB_per_s"]
        out["quantizer"]["frac_of_stream_read"] = gbs("quant") / rd["quant"]
        for name in decode:
            decode[name]["frac_of_stream_read"] = decode[name]["GB_per_s"] / rd[name]
    if args.cpu:
        progress("cpu baseline (oracle) ~%.0f s" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
