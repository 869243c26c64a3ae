"""Pins of the CPU oracle to things other than itself.

Each pin is a plain function of an ``oracle.Oracle`` that raises AssertionError when
the oracle disagrees with what the pages or the mathematics fix: printed values
(``tests/golden``), closed forms, invariants, exact rational arithmetic, brute force
on tiny inputs, and special cases that reduce to a numpy routine. The same pins run
against deliberately broken copies of the oracle (``test_oracle_mutants.py``), each
of which must fail at least one of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import workloads
from exact import rne_int, round_to_f16, round_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32_1EM10 = float(np.float32(1e-10))
# Half a quantization step plus the fp32 roundings of x / s and of s itself, in units
# of s: below 128 * 2^-24 + 2^-18 < 2^-15.
SLOP = 2.0 ** -15


def _rows(path):
    out = []
    for line in open(os.path.join(GOLDEN, path)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append([p.strip() for p in line.split(";")])
    return out


def _finite_halves():
    bits = np.arange(65536, dtype=np.uint16)
    h = bits.view(np.float16)
    return bits[np.isfinite(h)]


# ------------------------------------------------------------------ binary16

def pin_f16_decode_all(orc):
    """Every binary16 bit pattern decodes to numpy's float16 value."""
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.f16_bits_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_f16_encode_ties_and_roundtrip(orc):
    """Exact halves encode to themselves; midpoints between neighbours go to the even
    neighbour (computed exactly from the binary16 definition); random floats match the
    exact rational rounding."""
    bits = _finite_halves()
    vals = bits.view(np.float16).astype(np.float32)
    got = orc.f32_to_f16_bits(vals)
    # -0.0 and +0.0 both round-trip bit-exactly
    assert np.array_equal(got, bits)
    pos = np.sort(vals[(vals > 0)].astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)     # exact: 12 significant bits
    gm = orc.f32_to_f16_bits(mids).view(np.float16).astype(np.float64)
    rng = np.random.default_rng(7)
    pick = rng.choice(mids.size, 400, replace=False)
    for i in pick:
        assert gm[i] == round_to_f16(Fraction(float(mids[i]))), float(mids[i])
    # above the largest finite half by at least half an ulp -> inf
    assert orc.f32_to_f16_bits(np.array([65520.0], np.float32))[0] == 0x7C00
    assert orc.f32_to_f16_bits(np.array([65519.0], np.float32))[0] == 0x7BFF
    r = (rng.standard_normal(300) * np.exp2(rng.uniform(-26, 15, 300))).astype(np.float32)
    gr = orc.f32_to_f16_bits(r).view(np.float16).astype(np.float64)
    for v, g in zip(r, gr):
        assert g == round_to_f16(Fraction(float(v))), float(v)


# ---------------------------------------------------------- int8 quantizer

def pin_quant_golden_ties(orc):
    """Hand-derived tie cases (tests/golden/quant_ties.txt)."""
    for s_txt, x_txt, q_txt in _rows("quant_ties.txt"):
        x = np.array([float(v) for v in x_txt.split()], np.float32)[None, :]
        q_ref = np.array([int(v) for v in q_txt.split()], np.int8)
        q, s = orc.quant_rows_i8(x)
        assert float(s[0]) == float(s_txt), (s, s_txt)
        assert np.array_equal(q[0], q_ref), (q[0], q_ref)


def pin_quant_exact_rational(orc):
    """scale = round_f32(max(absmax, 1e-10) / 127) and q = rne(round_f32(x / scale)),
    clamped to [-127, 127], checked in exact rational arithmetic on sampled elements."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 300)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    x[2, :] = 0.0
    x[3, 5] = 7.0e-12          # tiny row absmax below the floor
    x[3, :5] = 0.0
    x[3, 6:] = 0.0
    q, s = orc.quant_rows_i8(x)
    for r in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[r])
        s_ref = round_to_f32(Fraction(max(a, F32_1EM10)) / 127)
        assert float(s[r]) == s_ref, (r, float(s[r]), s_ref)
        for c in rng.choice(x.shape[1], 60, replace=False):
            qt = rne_int(round_to_f32(Fraction(float(x[r, c])) / Fraction(s_ref)))
            qt = max(-127, min(127, qt))
            assert int(q[r, c]) == qt, (r, c)


def pin_quant_invariants(orc):
    """|q| <= 127; |x - q s| <= s/2 (+ the division's rounding); each row's absmax
    element maps to +-127; rows are quantized independently (per-row axis)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    x *= np.exp2(rng.integers(-12, 12, (32, 1))).astype(np.float32)   # very different row ranges
    x[:, 17] *= 20.0
    q, s = orc.quant_rows_i8(x)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + SLOP))
    am = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(np.abs(q[np.arange(32), am]).astype(int), np.full(32, 127))
    assert np.all(np.max(np.abs(q.astype(int)), axis=1) == 127)


def pin_quant_zero_row_floor(orc):
    """An all-zero row has absmax floored at 1e-10: scale = 1e-10/127, codes 0."""
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = -1.0
    q, s = orc.quant_rows_i8(x)
    assert float(s[0]) == round_to_f32(Fraction(F32_1EM10) / 127)
    assert not q[0].any()
    assert q[1, 3] == -127


def pin_quant_power_of_two_invariance(orc):
    """Scaling a row by 2^j scales its scale by 2^j exactly and leaves the codes alone."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q0, s0 = orc.quant_rows_i8(x)
    for j in (-7, -1, 3, 9):
        q1, s1 = orc.quant_rows_i8(x * np.float32(2.0 ** j))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** j))


def pin_quant_fp16_domain(orc):
    """Every finite fp16 value as an activation under several row absmax values:
    codes stay within [-127, 127] and within half a step of x / s (exact arithmetic
    on a sample, bound on all); fp16 rows decode exactly before quantizing."""
    vals = _finite_halves().view(np.float16)
    for amax in (np.float16(65504.0), np.float16(127.0), np.float16(1.0), np.float16(0.0078125)):
        row = vals[np.abs(vals.astype(np.float32)) <= np.float32(amax)]
        row = np.concatenate([[amax], row]).astype(np.float16)[None, :]
        q, s = orc.quant_rows_i8(row)
        xf = row.astype(np.float64)[0]
        sv = float(s[0])
        assert sv == round_to_f32(Fraction(float(amax)) / 127)
        assert q.min() >= -127 and q.max() <= 127
        assert np.all(np.abs(xf / sv - q[0]) <= 0.5 + SLOP)
        idx = np.random.default_rng(int(float(amax) * 8)).choice(row.shape[1], 200, replace=False)
        for c in idx:
            qt = rne_int(round_to_f32(Fraction(float(xf[c])) / Fraction(sv)))
            assert int(q[0, c]) == max(-127, min(127, qt))


def pin_quant_fp16_domain_exhaustive(orc):
    """Every finite fp16 activation under each of six row absmax values, every code
    checked: q = rne(fl32(x / s)). fl32 of a quotient is computed as the fp64 quotient
    rounded to fp32, which equals the directly rounded fp32 quotient because double
    rounding through 53 bits is innocuous for division at 24 bits (53 >= 2*24 + 2)."""
    vals = _finite_halves().view(np.float16)
    # the last four absmax values are ones where x * (127 / a) would round differently
    for amax in (65504.0, 1000.0, 127.0, 3.0, 1.0, 0.0078125,
                 0.947265625, 2.32421875, 1.4931640625, 0.1285400390625):
        amax16 = np.float16(amax)
        row = vals[np.abs(vals.astype(np.float32)) <= np.float32(amax16)]
        row = np.concatenate([[amax16], row]).astype(np.float16)[None, :]
        q, s = orc.quant_rows_i8(row)
        sv = round_to_f32(Fraction(float(amax16)) / 127)
        assert float(s[0]) == sv
        quot = (row[0].astype(np.float64) / sv).astype(np.float32).astype(np.float64)
        ref = np.clip(np.rint(quot), -127, 127).astype(np.int8)
        assert np.array_equal(q[0], ref), amax


def pin_int4_golden_ties(orc):
    """Hand-derived int4 tie cases (tests/golden/int4_ties.txt); one group of 8 padded
    with zeros to the group size 128 is still the same group absmax."""
    for s_txt, w_txt, q_txt in _rows("int4_ties.txt"):
        wv = [float(v) for v in w_txt.split()]
        w = np.zeros((1, 128), np.float32)
        w[0, :len(wv)] = wv
        packed, s16 = orc.quant_int4_group(w, 128)
        assert float(s16[0, 0]) == float(s_txt)
        q = orc.unpack_int4(packed, 128)[0, :len(wv)]
        assert q.tolist() == [int(v) for v in q_txt.split()], (q, q_txt)


def pin_per_tensor_is_one_row(orc):
    """Per-tensor quantization of a [R, C] array is per-row quantization of its flattening
    into one row of R*C (hotelren.com: one global absmax and one scale); the global argmax
    maps to +-127 and a row far below the maximum keeps small codes."""
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((6, 40)) * np.exp2(rng.integers(-6, 6, (6, 1)))).astype(np.float32)
    qt, st = orc.quant_tensor_i8(x)
    qr, sr = orc.quant_rows_i8(x.reshape(1, -1))
    assert np.array_equal(qt.reshape(1, -1), qr) and np.float32(st) == sr[0]
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(int(qt[i])) == 127
    assert np.float32(st) == np.float32(np.float32(np.abs(x).max()) / np.float32(127.0))


def pin_per_channel_beats_per_tensor(orc):
    """On weights whose column ranges vary (log-uniform sigma in [0.005, 0.5], the small
    W8A8 workload's law), per-output-channel scales give a weight MSE at least 5x below
    one per-tensor scale, and a smaller output error (2048ai.net §4, §6.2, qualitative)."""
    inp = workloads.draw(workloads.W8A8_SMALL)
    w = inp.w_nk
    qc, sc = orc.quant_weight_per_channel(w)
    qt, st = orc.quant_tensor_i8(w)
    wc = qc.astype(np.float64) * sc[:, None]
    wt = qt.astype(np.float64) * st
    mse_c = np.mean((wc - w) ** 2)
    mse_t = np.mean((wt - w) ** 2)
    assert mse_t >= 5.0 * mse_c, (mse_c, mse_t)
    x = inp.x.astype(np.float64)
    y = x @ w.T
    assert np.mean((x @ wc.T - y) ** 2) < np.mean((x @ wt.T - y) ** 2)


# ------------------------------------------------------------ integer GEMM

def pin_gemm_brute_force(orc):
    """int32 GEMM equals a Python-int triple loop on tiny non-square shapes."""
    rng = np.random.default_rng(21)
    for M, N, K in ((1, 1, 64), (3, 17, 64), (17, 3, 128), (5, 7, 192)):
        a = rng.integers(-127, 128, (M, K), dtype=np.int8)
        b = rng.integers(-127, 128, (N, K), dtype=np.int8)
        acc = orc.gemm_i32(a, b)
        al, bl = a.tolist(), b.tolist()
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(al[m][k] * bl[n][k] for k in range(K))


def pin_gemm_numpy_and_extremes(orc):
    """Equals numpy's int64 matmul of X and W (W given column-major); all +127 against all
    -127 gives -K * 127^2."""
    rng = np.random.default_rng(22)
    a = rng.integers(-127, 128, (37, 320), dtype=np.int8)
    b = rng.integers(-127, 128, (29, 320), dtype=np.int8)
    assert np.array_equal(orc.gemm_i32(a, b), a.astype(np.int64) @ b.astype(np.int64).T)
    K = 4096
    acc = orc.gemm_i32(np.full((2, K), 127, np.int8), np.full((3, K), -127, np.int8))
    assert np.all(acc == -K * 127 * 127)


# ---------------------------------------------------------------- epilogue

def pin_epilogue_special_and_bound(orc):
    """Unit scales and no bias give the accumulator itself; power-of-two scales and a
    dyadic bias are exact; in general the fp32 result lies within 4u of the exact value
    (relative to |acc xs ws| + |bias|), and the fp64 result within 4 * 2^-53."""
    rng = np.random.default_rng(31)
    acc = rng.integers(-(1 << 23), 1 << 23, (4, 6)).astype(np.int32)
    y32, y64 = orc.epilogue_w8a8(acc, np.ones(4, np.float32), np.ones(6, np.float32))
    assert np.array_equal(y32, acc.astype(np.float32)) and np.array_equal(y64, acc.astype(np.float64))
    # |acc| < 2^11, scales 2^-6..2^0 and bias a multiple of 2^-12 in [-1, 1]: every
    # intermediate is a multiple of 2^-12 below 2^12, i.e. exact in 24 bits
    acc = rng.integers(-(1 << 11), 1 << 11, (4, 6)).astype(np.int32)
    xs = np.exp2(rng.integers(-6, 1, 4)).astype(np.float32)
    ws = np.exp2(rng.integers(-6, 1, 6)).astype(np.float32)
    b = (rng.integers(-4096, 4097, 6) / 4096.0).astype(np.float32)
    y32, _ = orc.epilogue_w8a8(acc, xs, ws, b)
    for m in range(4):
        for n in range(6):
            assert Fraction(float(y32[m, n])) == (Fraction(int(acc[m, n])) * Fraction(float(xs[m]))
                                                   * Fraction(float(ws[n])) + Fraction(float(b[n])))
    acc = rng.integers(-66064384, 66064384, (5, 7)).astype(np.int32)
    xs = rng.uniform(1e-3, 1e-1, 5).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, 7).astype(np.float32)
    b = rng.standard_normal(7).astype(np.float32)
    y32, y64 = orc.epilogue_w8a8(acc, xs, ws, b)
    for m in range(5):
        for n in range(7):
            prod = Fraction(int(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
            exact = prod + Fraction(float(b[n]))
            mag = abs(prod) + abs(Fraction(float(b[n])))
            assert abs(Fraction(float(y32[m, n])) - exact) <= Fraction(4, 2 ** 24) * mag
            assert abs(Fraction(float(y64[m, n])) - exact) <= Fraction(4, 2 ** 53) * mag


def pin_w8a8_one_hot(orc):
    """X = e_k rows: x_scale = fl(1/127), xq = 127 e_k, acc[m, n] = 127 wq[k_m, n], and the
    layer output is within one quantization step of W[k_m, n] (+ bias)."""
    rng = np.random.default_rng(32)
    K, N = 128, 24
    w = (rng.standard_normal((N, K)) * rng.uniform(0.01, 1, (N, 1))).astype(np.float32)
    wq, ws = orc.quant_weight_per_channel(w)
    ks = np.array([0, 5, 77, 127])
    x = np.zeros((4, K), np.float32)
    x[np.arange(4), ks] = 1.0
    bias = rng.standard_normal(N).astype(np.float32)
    r = orc.linear_w8a8(x, wq, ws, bias)
    assert np.all(r["x_scale"] == np.float32(1.0) / np.float32(127.0))
    assert np.array_equal(r["xq"], (127 * x).astype(np.int8))
    assert np.array_equal(r["acc"], 127 * wq[:, ks].T.astype(np.int32))
    err = np.abs(r["y64"] - (w[:, ks].T.astype(np.float64) + bias))
    assert np.all(err <= 0.5 * ws[None, :] * 1.001)


# -------------------------------------------------------------- weight-only

def pin_w8a16_integer_special_case(orc):
    """Unit scales and no zero point: an fp GEMM with integer weights, equal to numpy's
    float64 matmul."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 256)).astype(np.float16)
    q = rng.integers(-127, 128, (40, 256), dtype=np.int8)
    y = orc.w8a16_f64(x, q, np.ones(40, np.float32))
    ref = x.astype(np.float64) @ q.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)


def pin_w8a16_one_hot(orc):
    """x = e_k: y[n] = (q[k, n] - z[b(k), n]) * s[b(k), n] exactly, for per-channel and
    block-64 zero-point layouts (pins the scale/zero indexing and the sign of z)."""
    rng = np.random.default_rng(42)
    N, K = 10, 256
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s = rng.uniform(1e-3, 1e-1, N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    ks = [0, 63, 64, 200]
    x = np.zeros((len(ks), K), np.float16)
    x[np.arange(len(ks)), ks] = 1.0
    y = orc.w8a16_f64(x, q, s, bias=bias)
    for i, k in enumerate(ks):
        for n in range(N):
            assert y[i, n] == float(Fraction(int(q[n, k])) * Fraction(float(s[n])) + Fraction(float(bias[n])))
    u = rng.integers(0, 256, (N, K), dtype=np.uint8)
    sb = rng.uniform(1e-3, 1e-1, (N, K // 64)).astype(np.float32)
    zb = rng.integers(0, 256, (N, K // 64), dtype=np.uint8)
    y = orc.w8a16_f64(x, u, sb, zero_point=zb, group_size=64)
    for i, k in enumerate(ks):
        for n in range(N):
            assert y[i, n] == float((int(u[n, k]) - int(zb[n, k // 64])) * Fraction(float(sb[n, k // 64])))


def pin_block_asym_quantizer(orc):
    """Block-64 asymmetric uint8 (zingnex.cn steps 1-2): scale = (max-min)/255 (fp32),
    the block minimum codes to 0 exactly, the maximum to 254 or 255, and every weight
    comes back within half a step: |w - (q - zp) s| <= s/2 (+ rounding)."""
    inp = workloads.draw(workloads.with_shape(workloads.W8A16_BLOCK, 1, 512, 48))
    w = inp.w_nk
    q, s, z = orc.quant_block_asym_u8(w, 64)
    blocks = w.reshape(48, 8, 64)
    qb = q.reshape(48, 8, 64).astype(np.int64)
    mn, mx = blocks.min(-1), blocks.max(-1)
    for n in range(0, 48, 5):
        for b in range(8):
            assert float(s[n, b]) == round_to_f32(Fraction(round_to_f32(Fraction(float(mx[n, b])) - Fraction(float(mn[n, b])))) / 255)
    assert np.all(qb[np.arange(48)[:, None], np.arange(8)[None, :], blocks.argmin(-1)] == 0)
    assert np.all(np.isin(qb[np.arange(48)[:, None], np.arange(8)[None, :], blocks.argmax(-1)], (254, 255)))
    deq = (qb - z[:, :, None].astype(np.int64)) * s[:, :, None].astype(np.float64)
    assert np.all(np.abs(deq - blocks) <= s[:, :, None] * (0.5 + 2.0 ** -16))


def pin_int4_pack_layout(orc):
    """Eight two's-complement nibbles per int32 along K, element k%8 = j in bits
    [4j, 4j+3]: the oracle's unpack inverts an independent numpy pack, over all 16 values
    at all 8 positions."""
    N, K = 16, 128
    q = np.empty((N, K), np.int64)
    for n in range(N):
        q[n] = (np.arange(K) + n) % 16 - 8
    nib = (q & 0xF).astype(np.uint64).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), np.uint64)
    for j in range(8):
        words |= nib[:, :, j] << np.uint64(4 * j)
    packed = words.astype(np.uint32).view(np.int32)
    assert np.array_equal(orc.unpack_int4(packed, K).astype(np.int64), q)


def pin_int4_quantizer(orc):
    """int4 group quantizer (xdnf.cn §5.1, scale = absmax/7, stored fp16): the scale is
    the fp16 rounding of the fp32 quotient, each group's absmax element codes to +-7,
    codes stay in [-8, 7] and every weight is within half a step of q * s16."""
    inp = workloads.draw(workloads.with_shape(workloads.W4A16_GROUP, 1, 512, 40))
    w = inp.w_nk
    packed, s16 = orc.quant_int4_group(w, 128)
    q = orc.unpack_int4(packed, 512).astype(np.int64).reshape(40, 4, 128)
    g = w.reshape(40, 4, 128)
    a = np.abs(g).max(-1)
    for n in range(0, 40, 3):
        for b in range(4):
            s32 = round_to_f32(Fraction(float(a[n, b])) / 7)
            assert float(s16[n, b]) == round_to_f16(Fraction(s32))
    sv = s16.astype(np.float64)[:, :, None]
    am = np.abs(g).argmax(-1)
    assert np.all(np.abs(q[np.arange(40)[:, None], np.arange(4)[None, :], am]) == 7)
    assert q.min() >= -8 and q.max() <= 7
    assert np.all(np.abs(g - q * sv) <= sv * (0.5 + 2.0 ** -16))


def pin_w4a16_one_hot(orc):
    """x = e_k: y[n] = q[k, n] * s16[k // group, n] exactly (pins nibble order, sign
    extension and group indexing)."""
    rng = np.random.default_rng(51)
    N, K, G = 12, 512, 128
    w = rng.standard_normal((N, K)).astype(np.float32)
    packed, s16 = orc.quant_int4_group(w, G)
    q = orc.unpack_int4(packed, K)
    ks = [0, 1, 7, 8, 127, 128, 300, 511]
    x = np.zeros((len(ks), K), np.float16)
    x[np.arange(len(ks)), ks] = 1.0
    y = orc.w4a16_f64(x, packed, s16, G)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], q[:, k].astype(np.float64) * s16[:, k // G].astype(np.float64))


def pin_footprint_golden(orc):
    """The pages' printed footprints (tests/golden/footprint.txt) follow from the code
    formats' storage: 1 byte per int8 code, 4 bytes per 8 int4 codes."""
    w = np.random.default_rng(61).standard_normal((8, 256)).astype(np.float32)
    q8, _ = orc.quant_weight_per_channel(w)
    p4, _ = orc.quant_int4_group(w, 128)
    bytes_per = {16: 2.0, 8: q8.nbytes / w.size, 4: p4.nbytes / w.size}
    for params, bits, printed, unit in _rows("footprint.txt"):
        size = float(params) * bytes_per[int(bits)] / (2 ** 30 if unit == "GiB" else 1e9)
        nd = len(printed.split(".")[1]) if "." in printed else 0
        assert abs(size - float(printed)) <= 0.5 * 10 ** -nd + 1e-9, (params, bits, size, printed)


def pin_asym_quant_rows(orc):
    """Asymmetric rows (hotelren.com per_channel_quant_int8, asymmetric branch): the row
    minimum codes to -128 and the maximum to 127; every element dequantizes to within half
    a step, |s (q - z) - x| <= s (1/2 + 2^-14 (|x|/s + 256)) for fp32's roundings; the zero
    point is 255 (-lo) / (hi - lo) - 128 up to fp32 rounding, not rounded to an integer; a
    constant row takes the 1e-8 scale floor, codes -128 and dequantizes to itself."""
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((64, 300)) * np.exp2(rng.integers(-6, 6, (64, 1)))
         + rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    q, s, z = orc.quant_rows_i8_asym(x)
    r = np.arange(64)
    assert np.all(q[r, x.argmin(1)] == -128) and np.all(q[r, x.argmax(1)] == 127)
    sd = s.astype(np.float64)[:, None]
    deq = sd * (q.astype(np.float64) - z.astype(np.float64)[:, None])
    assert np.all(np.abs(deq - x) <= sd * (0.5 + 2.0 ** -14 * (np.abs(x) / sd + 256)))
    lo, hi = x.min(1).astype(np.float64), x.max(1).astype(np.float64)
    zr = 255.0 * (-lo) / (hi - lo) - 128.0
    assert np.all(np.abs(z - zr) <= 1e-4 * (1 + np.abs(zr)))
    frac = np.abs(z - np.round(z))
    assert (frac > 0.01).mean() > 0.5          # the zero point is kept as a float
    c = np.full((3, 40), [[0.75], [-2.5], [1e-3]], np.float32)
    qc, sc, zc = orc.quant_rows_i8_asym(c)
    assert np.all(qc == -128) and np.all(sc == np.float32(1e-8))
    dc = sc.astype(np.float64) * (-128.0 - zc.astype(np.float64))
    assert np.allclose(dc, c[:, 0], rtol=1e-5, atol=0)


def pin_asym_quant_relu_rows(orc):
    """A row with minimum 0 whose values are exact multiples k of a power-of-two step with
    k up to 255: the scale is the step, the zero point is -128 and the codes are k - 128."""
    rng = np.random.default_rng(82)
    for e in (-3, 0, 5):
        k = rng.permutation(np.concatenate([[0, 255], rng.integers(0, 256, 98)]))
        row = (k * 2.0 ** e).astype(np.float32)[None, :]
        q, s, z = orc.quant_rows_i8_asym(row)
        assert s[0] == np.float32(2.0 ** e) and z[0] == -128.0
        assert np.array_equal(q[0].astype(np.int64), k - 128)


def pin_asym_layer(orc):
    """The asymmetric layer against exact rational arithmetic on tiny inputs, and against
    numpy's fp64 product of the dequantized operands, s_x (q_x - z_x) @ (s_w q_w)^T + b;
    column sums against numpy."""
    rng = np.random.default_rng(83)
    M, N, K = 3, 4, 8
    xq = rng.integers(-128, 128, (M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xs = rng.uniform(0.01, 0.1, M).astype(np.float32)
    xz = rng.uniform(-100, 100, M).astype(np.float32)
    ws = rng.uniform(0.01, 0.1, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y = orc.w8a8_asym_f64(xq, xs, xz, wq, ws, b)
    for m in range(M):
        for n in range(N):
            t = sum((Fraction(int(xq[m, k])) - Fraction(float(xz[m]))) * int(wq[n, k]) for k in range(K))
            exact = t * Fraction(float(xs[m])) * Fraction(float(ws[n])) + Fraction(float(b[n]))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10 ** 12) * (abs(exact) + 1)
    M, N, K = 50, 60, 300
    xq = rng.integers(-128, 128, (M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xs, xz = rng.uniform(0.01, 0.1, M).astype(np.float32), rng.uniform(-128, 127, M).astype(np.float32)
    ws, b = rng.uniform(0.01, 0.1, N).astype(np.float32), rng.standard_normal(N).astype(np.float32)
    xd = xs.astype(np.float64)[:, None] * (xq.astype(np.float64) - xz.astype(np.float64)[:, None])
    wd = ws.astype(np.float64)[:, None] * wq.astype(np.float64)
    ref = xd @ wd.T + b.astype(np.float64)[None, :]
    assert np.allclose(orc.w8a8_asym_f64(xq, xs, xz, wq, ws, b), ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(orc.column_sums_i8(wq), wq.astype(np.int64).sum(1))


def _e4m3_table(orc):
    vals = orc.e4m3_decode(np.arange(256))
    return vals


def pin_e4m3_format(orc):
    """The OCP E4M3 format's fixed points: 1.0 is 0x38, the largest finite value 448 is
    0x7E, the smallest normal 2^-6 is 0x08, the smallest subnormal 2^-9 is 0x01, NaN is
    exactly 0x7F and 0xFF, 0x80 is -0, the sign bit negates, the 127 non-negative finite
    codes increase strictly, and consecutive normals of one binade are 2^(e-10) apart."""
    v = _e4m3_table(orc)
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)
    for e in range(1, 15):
        b = pos[8 * e:8 * e + 8]
        assert np.allclose(np.diff(b), 2.0 ** (e - 10), rtol=0, atol=0)


def pin_e4m3_encode(orc):
    """Encoding is round to nearest with ties to an even mantissa: every midpoint between
    consecutive finite values goes to the even code, and random values land within half a
    spacing of their value (checked by bisection of the sorted value table)."""
    v = _e4m3_table(orc)
    pos = v[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    got = orc.e4m3_encode(mids.astype(np.float32))
    want = np.where(np.arange(1, 127) % 2 == 0, np.arange(1, 127), np.arange(0, 126))
    assert np.array_equal(got.astype(np.int64), want)
    assert np.array_equal(orc.e4m3_encode(-mids.astype(np.float32)).astype(np.int64), want | 0x80)
    x = np.random.default_rng(101).uniform(-448, 448, 4000).astype(np.float32)
    x[:1000] *= np.float32(2.0 ** -8)
    q = orc.e4m3_encode(x)
    a = np.abs(x.astype(np.float64))
    i = np.clip(np.searchsorted(pos, a), 1, 126)
    near = np.minimum(np.abs(pos[i] - a), np.abs(pos[i - 1] - a))
    assert np.all(np.abs(np.abs(v[q]) - a) <= near * (1 + 1e-12))
    assert np.all((q >> 7) == np.signbit(x))


def pin_e4m3_quant_and_layer(orc):
    """Per-row fp8: each row's absmax element codes to +-448 and every normal-range element
    dequantizes within 2^-4 relative (three mantissa bits); an all-zero row takes the floor
    scale 1e-10/448. The fp8 layer equals numpy's fp64 product of the decoded codes, and its
    magnitude bounds |y - bias|."""
    rng = np.random.default_rng(102)
    x = (rng.standard_normal((40, 256)) * np.exp2(rng.integers(-8, 8, (40, 1)))).astype(np.float32)
    x[3] = 0
    q, s = orc.quant_rows_e4m3(x)
    v = _e4m3_table(orc)
    r = np.arange(40)
    am = np.abs(x).argmax(1)
    assert np.all(np.abs(v[q[r, am]][r != 3]) == 448.0)
    assert s[3] == np.float32(np.float32(1e-10) / np.float32(448.0)) and np.all(q[3] == 0)
    deq = v[q] * s.astype(np.float64)[:, None]
    normal = np.abs(x) >= 2.0 ** -6 * s[:, None]
    assert np.all(np.abs(deq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    wq, ws = orc.quant_rows_e4m3(rng.standard_normal((30, 256)).astype(np.float32))
    b = rng.standard_normal(30).astype(np.float32)
    y, mag = orc.gemm_e4m3_f64(q, s, wq, ws, b)
    ref = (v[q] * s.astype(np.float64)[:, None]) @ (v[wq] * ws.astype(np.float64)[:, None]).T + b[None, :]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-300)
    assert np.all(np.abs(y - b[None, :]) <= mag * (1 + 1e-12) + 1e-300)


# Standard normal distribution function at tabulated points (values from a normal table,
# to 16 significant digits); 1.959963984540054 is the 0.975 quantile.
PHI_TABLE = {-3.0: 0.001349898031630095, -0.5: 0.3085375387259869, 0.0: 0.5,
             1.0: 0.8413447460685429, 2.0: 0.9772498680518208, 1.959963984540054: 0.975}


def pin_activation_values(orc):
    """GELU(y) = y Phi(y) at tabulated points of Phi; SiLU(y) = y sigmoid(y) where sigmoid
    is rational (sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4) or
    e / (1 + e) at 1; act 0 is the identity."""
    ys = np.array(sorted(PHI_TABLE))
    got = orc.activation_f64(ys, 1)
    want = ys * np.array([PHI_TABLE[v] for v in ys])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-300), (got, want)
    s = np.array([0.0, np.log(3.0), -np.log(3.0), 1.0])
    got = orc.activation_f64(s, 2)
    want = s * np.array([0.5, 0.75, 0.25, np.e / (1.0 + np.e)])
    assert np.allclose(got, want, rtol=1e-14, atol=0.0), (got, want)
    r = np.random.default_rng(71).standard_normal(64) * 5
    assert np.array_equal(orc.activation_f64(r, 0), r)


def pin_activation_invariants(orc):
    """For both activations act(y) - act(-y) = y (Phi(-y) = 1 - Phi(y) and
    sigmoid(-y) = 1 - sigmoid(y)); act(y) -> y for large y and -> 0 for very negative y;
    both are increasing for y >= 0."""
    y = np.random.default_rng(72).standard_normal(4096) * 4
    for act in (1, 2):
        a, b = orc.activation_f64(y, act), orc.activation_f64(-y, act)
        assert np.allclose(a - b, y, rtol=0, atol=1e-12 * (1 + np.abs(y)).max())
        big = orc.activation_f64(np.array([40.0, -40.0]), act)
        assert abs(big[0] - 40.0) < 1e-12 and abs(big[1]) < 1e-12
        pos = orc.activation_f64(np.linspace(0, 10, 1001), act)
        assert np.all(np.diff(pos) > 0)


def pin_wonly_f32seq(orc):
    """The fp32 k-order sum: equal to the fp64 product where every partial sum is exact
    (small integer activations and codes, power-of-two scales, block zero points); equal to
    numpy's float32 cumulative sum of the float32 products in k order elsewhere; and within
    K * 2^-24 * sum |terms| of the fp64 value."""
    rng = np.random.default_rng(93)
    M, K, N = 3, 128, 5
    x = rng.integers(-8, 9, (M, K)).astype(np.float32)
    q = rng.integers(0, 256, (N, K)).astype(np.uint8)
    z = rng.integers(0, 256, (N, K // 64)).astype(np.uint8)
    s = np.exp2(rng.integers(-4, 2, (N, K // 64))).astype(np.float32)
    y32 = orc.w8a16_f32seq(x, q, s, z, 64)
    assert np.array_equal(y32.astype(np.float64), orc.w8a16_f64(x, q, s, z, 64))
    x = rng.standard_normal((M, K)).astype(np.float32)
    q8 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s8 = rng.uniform(0.001, 0.01, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y32 = orc.w8a16_f32seq(x, q8, s8, None, 0, b)
    w = (q8.astype(np.float32) * s8[:, None]).astype(np.float32)
    for m in range(M):
        for n in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(x[m, k] * w[n, k]))
            assert y32[m, n] == np.float32(acc + b[n]), (m, n)
    y64 = orc.w8a16_f64(x, q8, s8, None, 0, b)
    terms = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T + np.abs(b)
    assert np.all(np.abs(y32 - y64) <= (K + 2) * 2.0 ** -24 * terms + 1e-9 * terms)


# ------------------------------------------------------- re-quantization of Y

def pin_requant_golden_ties(orc):
    """Hand-derived codes for exact quotients on ties, the clamp and scales that are not
    powers of two (tests/golden/requant_ties.txt), with one scale for the whole output and
    the same scale repeated per channel."""
    for s_txt, y_txt, q_txt in _rows("requant_ties.txt"):
        y = np.array([float(v) for v in y_txt.split()], np.float32)[None, :]
        q_ref = np.array([int(v) for v in q_txt.split()], np.int8)
        assert np.array_equal(orc.requant_i8(y, np.float32(s_txt))[0], q_ref), s_txt
        per_channel = np.full(y.shape[1], np.float32(s_txt), np.float32)
        assert np.array_equal(orc.requant_i8(y, per_channel)[0], q_ref), s_txt


def pin_requant_exact_rational(orc):
    """q = clamp(rne(round_f32(y / s[n])), -127, 127) in exact rational arithmetic, with a
    different scale per output channel (so a scale taken from the wrong axis fails) and
    values spanning the clamp."""
    rng = np.random.default_rng(91)
    M, N = 7, 33
    s = (np.exp2(rng.uniform(-12, 4, N)) * rng.uniform(1, 2, N)).astype(np.float32)
    y = (rng.standard_normal((M, N)) * s[None, :] * np.float32(60.0)).astype(np.float32)
    q = orc.requant_i8(y, s)
    for m in range(M):
        for n in range(N):
            t = rne_int(round_to_f32(Fraction(float(y[m, n])) / Fraction(float(s[n]))))
            assert int(q[m, n]) == max(-127, min(127, t)), (m, n)
    assert (np.abs(q) == 127).any() and (np.abs(q) < 127).any()


def pin_channel_scales(orc):
    """Calibrated scales: s[n] = round_f32(max(max_m |y[m, n]|, 1e-10) / 127) exactly, per
    column (not per row); an all-zero channel gets the floor; requantized with its own
    scales, each channel's largest |y| maps to +-127 and every code is within half a step."""
    rng = np.random.default_rng(92)
    M, N = 9, 12
    y = (rng.standard_normal((M, N)) * np.exp2(rng.integers(-8, 8, (1, N)))).astype(np.float32)
    y[:, 4] = 0.0
    s = orc.channel_scales(y)
    for n in range(N):
        a = max(abs(float(v)) for v in y[:, n])
        assert float(s[n]) == round_to_f32(Fraction(max(a, F32_1EM10)) / 127), n
    q = orc.requant_i8(y, s)
    for n in range(N):
        if n != 4:
            m = int(np.argmax(np.abs(y[:, n])))
            assert abs(int(q[m, n])) == 127, n
    assert np.all(q[:, 4] == 0)
    err = np.abs(q.astype(np.float64) * s[None, :] - y.astype(np.float64))
    assert np.all(err <= s[None, :].astype(np.float64) * (0.5 + SLOP))


# ------------------------------------- quotient reading x / s in every quantizer
#
# The codes of every quantizer are round(x / s) with x / s the correctly rounded fp32
# quotient. The multiply by a rounded reciprocal, x * round_f32(1 / s), agrees with it
# except near ties, so these pins put many exact ties x = (j + 1/2) s at scales that are
# not powers of two (where round_f32(1 / s) is inexact) and check every code.

# Odd-significand scales (not powers of two) and power-of-two multiples of them.
TIE_SCALES = (0.875, 0.9375, 0.8125, 0.875 * 2.0 ** -6, 0.9375 * 2.0 ** 5, 0.8125 * 2.0 ** -11)


def _f32(fr) -> Fraction:
    return Fraction(round_to_f32(Fraction(fr)))


def pin_asym_golden_ties(orc):
    """Hand-derived asymmetric codes at scale 0.875 with integer zero points
    (tests/golden/asym_ties.txt)."""
    for s_txt, z_txt, x_txt, q_txt in _rows("asym_ties.txt"):
        x = np.array([float(v) for v in x_txt.split()], np.float32)[None, :]
        q, s, z = orc.quant_rows_i8_asym(x)
        assert float(s[0]) == float(s_txt) and float(z[0]) == float(z_txt), (s, z)
        assert q[0].tolist() == [int(v) for v in q_txt.split()], (q[0], q_txt)


def _asym_ref_row(row):
    """Exact-rational evaluation of the asymmetric reading on one fp32 row: (codes, s, z)."""
    lo, hi = Fraction(float(min(row))), Fraction(float(max(row)))
    s = _f32(_f32(hi - lo) / 255)
    if s < Fraction(float(np.float32(1e-8))):
        s = Fraction(float(np.float32(1e-8)))
    z = _f32(_f32(-lo / s) - 128)
    q = [max(-128, min(127, rne_int(_f32(_f32(Fraction(float(v)) / s) + z)))) for v in row]
    return q, float(s), float(z)


def pin_asym_exact_rational(orc):
    """Asymmetric per-row codes, scales and zero points against exact rational arithmetic
    of the reading: s = fl(fl(hi - lo) / 255) (floor 1e-8), z = fl(fl(-lo / s) - 128),
    q = clamp(rne(fl(fl(x / s) + z)), -128, 127). Every code of rows built from exact ties
    (j + 1/2) s, with the row minimum at -j0 s so that the zero point is j0 - 128, and
    sampled codes of random rows."""
    rows = []
    for s in TIE_SCALES:
        for j0 in (0, 128, 250, 37):
            j = np.arange(-j0, 255 - j0)
            rows.append(np.concatenate([[-j0 * s, (255 - j0) * s], (j[:-1] + 0.5) * s]))
    width = max(len(r) for r in rows)
    x = np.array([np.resize(r, width) for r in rows], np.float32)
    q, s, z = orc.quant_rows_i8_asym(x)
    for i, r in enumerate(x):
        qr, sr, zr = _asym_ref_row(r)
        assert float(s[i]) == sr and float(z[i]) == zr, (i, float(s[i]), sr, float(z[i]), zr)
        assert q[i].tolist() == qr, i
    rng = np.random.default_rng(84)
    x = (rng.standard_normal((8, 200)) * np.exp2(rng.integers(-9, 9, (8, 1)))
         + rng.uniform(-2, 2, (8, 1))).astype(np.float32)
    q, s, z = orc.quant_rows_i8_asym(x)
    for i, r in enumerate(x):
        qr, sr, zr = _asym_ref_row(r)
        assert float(s[i]) == sr and float(z[i]) == zr, i
        assert q[i].tolist() == qr, i


def pin_block_asym_golden_ties(orc):
    """Hand-derived block-64 uint8 codes at scale 0.875, including a zero point that is a
    tie (tests/golden/block_asym_ties.txt)."""
    for s_txt, z_txt, w_txt, q_txt in _rows("block_asym_ties.txt"):
        wv = [float(v) for v in w_txt.split()]
        w = np.full((1, 64), wv[0], np.float32)
        w[0, :len(wv)] = wv
        q, s, z = orc.quant_block_asym_u8(w, 64)
        assert float(s[0, 0]) == float(s_txt) and int(z[0, 0]) == int(z_txt), (s, z)
        assert q[0, :len(wv)].tolist() == [int(v) for v in q_txt.split()], (q[0, :len(wv)], q_txt)


def _block_ref(block):
    """Exact-rational evaluation of the block-asymmetric reading on one block: (codes, s, zp)."""
    mn, mx = Fraction(float(min(block))), Fraction(float(max(block)))
    s = _f32(_f32(mx - mn) / 255)
    if s < Fraction(float(np.float32(1e-8))):
        s = Fraction(float(np.float32(1e-8)))
    zp = max(0, min(255, rne_int(_f32(-mn / s))))
    q = [max(0, min(255, rne_int(_f32(Fraction(float(v)) / s)) + zp)) for v in block]
    return q, float(s), zp


def pin_block_asym_exact_rational(orc):
    """Block-64 uint8 codes, scales and zero points against exact rational arithmetic of
    the reading: s = fl(fl(max - min) / 255) (floor 1e-8), zp = clamp(rne(fl(-min / s)),
    0, 255), q = clamp(rne(fl(w / s)) + zp, 0, 255). Every code of blocks of exact ties
    (j + 1/2) s (the minimum at -m0 s, with m0 an integer or itself a tie) and of blocks
    of a workload's weights."""
    rng = np.random.default_rng(85)
    blocks = []
    for s in TIE_SCALES:
        for m0 in (96, 96.5, 200, 200.5, 250):
            lo, hi = -m0 * s, (255 - m0) * s
            j = rng.choice(np.arange(-int(m0), int(254 - m0)), 62, replace=False)
            blocks.append(np.concatenate([[lo, hi], (j + 0.5) * s]))
    w = np.array(blocks, np.float32).reshape(-1, 128)     # two blocks per row
    inp = workloads.draw(workloads.with_shape(workloads.W8A16_BLOCK, 1, 128, 4))
    w = np.concatenate([w, inp.w_nk], 0)
    q, s, z = orc.quant_block_asym_u8(w, 64)
    for n in range(w.shape[0]):
        for b in range(2):
            qr, sr, zr = _block_ref(w[n, 64 * b:64 * b + 64])
            assert float(s[n, b]) == sr and int(z[n, b]) == zr, (n, b)
            assert q[n, 64 * b:64 * b + 64].tolist() == qr, (n, b)


def pin_int4_exact_rational(orc):
    """int4 group codes against exact rational arithmetic of the reading:
    s16 = fp16(fl(max(a, 7 * 2^-24) / 7)), q = clamp(rne(fl(w / s16)), -8, 7). Every code of
    groups of exact ties (j + 1/2) s16 with absmax 7 s16 at scales that are not powers of
    two, and of a workload's groups."""
    rng = np.random.default_rng(86)
    groups = []
    for s in TIE_SCALES:
        for _ in range(2):
            j = rng.integers(-7, 7, 127)          # |(j + 1/2) s| <= 6.5 s < 7 s
            groups.append(rng.permutation(np.concatenate([[7 * s * rng.choice([-1, 1])], (j + 0.5) * s])))
    w = np.array(groups, np.float32)
    w = np.concatenate([w, workloads.draw(workloads.with_shape(workloads.W4A16_GROUP, 1, 128, 6)).w_nk], 0)
    packed, s16 = orc.quant_int4_group(w, 128)
    q = orc.unpack_int4(packed, 128)
    floor_a = Fraction(7) * Fraction(1, 2 ** 24)
    for n in range(w.shape[0]):
        a = max(Fraction(abs(float(v))) for v in w[n])
        sr = Fraction(round_to_f16(_f32(max(a, floor_a) / 7)))
        assert Fraction(float(s16[n, 0])) == sr, n
        qr = [max(-8, min(7, rne_int(_f32(Fraction(float(v)) / sr)))) for v in w[n]]
        assert q[n].tolist() == qr, n


def pin_e4m3_golden_ties(orc):
    """Hand-derived E4M3 codes at scale 0.875, on midpoints between E4M3 values
    (tests/golden/e4m3_ties.txt)."""
    for s_txt, x_txt, q_txt in _rows("e4m3_ties.txt"):
        x = np.array([float(v) for v in x_txt.split()], np.float32)[None, :]
        q, s = orc.quant_rows_e4m3(x)
        assert float(s[0]) == float(s_txt), s
        assert q[0].tolist() == [int(v, 16) for v in q_txt.split()], ([hex(v) for v in q[0]], q_txt)


def _e4m3_code_exact(t: Fraction, negative: bool) -> int:
    """The E4M3 code of the value nearest to t (|t| <= 448), ties to the even mantissa,
    from the format's definition: spacing 2^-9 below 2^-6, else 2^(E-3) in [2^E, 2^(E+1))."""
    a = abs(t)
    if a < Fraction(1, 64):
        quantum = Fraction(1, 512)
    else:
        E = 0
        while Fraction(2) ** E > a:
            E -= 1
        while Fraction(2) ** (E + 1) <= a:
            E += 1
        quantum = Fraction(2) ** (E - 3)
    n = rne_int(a / quantum)
    v = n * quantum
    sign = 0x80 if negative else 0
    if v < Fraction(1, 64):
        return sign | int(v * 512)                      # exponent field 0: m / 8 * 2^-6
    E = 0
    while Fraction(2) ** E > v:
        E -= 1
    while Fraction(2) ** (E + 1) <= v:
        E += 1
    m = int((v / Fraction(2) ** E - 1) * 8)
    return sign | ((E + 7) << 3) | m


def pin_e4m3_exact_rational(orc):
    """Per-row E4M3 codes against exact rational arithmetic of the reading:
    s = fl(max(a, 1e-10) / 448), t = clamp(fl(x / s), -448, 448), code = the nearest E4M3
    value with ties to the even mantissa (a negative t keeps the sign bit). Every code of
    rows whose quotients are midpoints and values of E4M3 in every binade, at scales that
    are not powers of two, and of random rows."""
    pos = [Fraction(m, 512) for m in range(8)] + \
          [Fraction(2) ** (e - 7) * (1 + Fraction(m, 8)) for e in range(1, 16) for m in range(8)][:-1]
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    rows = []
    for s in TIE_SCALES:
        vals = [448 * s] + [float(v) * s for v in mids] + [-float(v) * s for v in mids[::3]] + \
               [float(v) * s for v in pos[1::5]]
        rows.append(vals)
    width = max(len(r) for r in rows)
    x = np.array([np.resize(r, width) for r in rows], np.float32)
    rng = np.random.default_rng(87)
    xr = (rng.standard_normal((6, width)) * np.exp2(rng.integers(-10, 10, (6, 1)))).astype(np.float32)
    xr[:, :40] *= np.float32(2.0 ** -9)          # subnormal E4M3 quotients
    x = np.concatenate([x, xr], 0)
    q, s = orc.quant_rows_e4m3(x)
    f1e10 = Fraction(float(np.float32(1e-10)))
    for i, r in enumerate(x):
        a = max(Fraction(abs(float(v))) for v in r)
        sr = _f32(max(a, f1e10) / 448)
        assert Fraction(float(s[i])) == sr, i
        for c, v in enumerate(r):
            t = _f32(Fraction(float(v)) / sr)
            t = max(Fraction(-448), min(Fraction(448), t))
            assert int(q[i, c]) == _e4m3_code_exact(t, bool(np.signbit(v))), (i, c, float(v))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
