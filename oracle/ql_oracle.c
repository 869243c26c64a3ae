/*
 * ql_oracle.c -- CPU oracle for the symmetric per-channel quantized linear layer
 *
 *     Y = (x_scale (.) Xq) @ (w_scale (.) Wq) + bias
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or loads
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do. It shares no code, header, table or helper with the HIP library.
 *
 * Every function is a plain loop written from the definitions on the pages:
 *   - linear quantization q = round(x/s) + z, x ~ s(q - z); symmetric z = 0 with
 *     codes in [-127, 127]             quant67.com ch.17 "量化与多精度算子", §二
 *   - scale = max|x| / 127              2048ai.net Llama-2-7B INT8 write-up, §2.2
 *   - per-row absmax, floor 1e-10, round-to-nearest-even (torch.round)
 *                                       hotelren.com "量化算法的本质", per_channel_quant_int8
 *   - Y = (x_scale*X) @ (w_scale*W) + bias, X [M,K] row-major, W [K,N] column-major
 *                                       hotelren.com, "W8A8矩阵乘法"
 *   - int32 accumulation, dequantize at write-back
 *                                       2048ai.net §5.4; quant67.com §四, §六
 *   - block-64 asymmetric uint8: scale = (max-min)/255, zero = round(-min/scale),
 *     q = round(w/scale) + zero          zingnex.cn "从零实现大语言模型 INT8 量化", 核心量化流程
 *   - int4 weights, scale = max|w| / 7, unpack then (q - zp) * scale
 *                                       xdnf.cn INT4/FP16 mixed GEMM on CANN TBE, §3.2, §5.1
 *
 * Precision: the quantizers decide integer codes in fp32, the precision the pages
 * compute scales in (x.float()); the integer GEMM is exact; the W8A8 epilogue is
 * given both in fp32 (left to right, no fused multiply-add: built with
 * -ffp-contract=off) and in fp64; the weight-only products are fp64.
 *
 * Readings taken where the pages are silent or disagree (all also listed in the
 * design notes): round half to even everywhere; the code is x / s with
 * s = absmax/127 (two correctly rounded fp32 divisions, never x * (127/absmax));
 * symmetric clamp [-127, 127]; an all-zero row gets absmax floored at 1e-10;
 * per-channel weight scales are per output column n; block-asymmetric zero points
 * are clamped to [0, 255] and added as integers, the block scale floored at 1e-8;
 * int4 codes are two's complement, eight per int32 along K, element k%8 = j in
 * bits [4j, 4j+3]; the int4 group scale is rounded to fp16 and codes are taken with
 * the stored fp16 scale; its absmax floor is 7 * 2^-24 so that the fp16 scale is
 * never zero.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "ql_oracle.h"

/* ---------------------------------------------------------------- binary16 */
/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */

float oracle_f16_to_f32(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return sign | 0x7e00u;
    if (isinf(x))
        return sign | 0x7c00u;
    double a = fabs((double)x);
    if (a < 0x1p-14) {
        /* subnormal range, spacing 2^-24; a result of 1024 is the smallest normal */
        double r = nearbyint(a * 0x1p24);
        return sign | (uint16_t)r;
    }
    int e2;
    frexp(a, &e2);                 /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    double r = nearbyint(ldexp(a, 10 - E));   /* significand in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00u;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

void oracle_f16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_f16(x[i]);
}

/* ------------------------------------------------------- symmetric int8 */

/* One symmetric int8 quantization of a contiguous vector v[0..n):
 *   a = max |v|,  s = max(a, 1e-10) / 127 (fp32),  q = clamp(rne(v / s), -127, 127). */
static float quant_vec_i8(const float* v, int64_t n, int8_t* q)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float t = fabsf(v[i]);
        if (t > a)
            a = t;
    }
    const float floor_a = 1e-10f;
    float s = (a > floor_a ? a : floor_a) / 127.0f;
    for (int64_t i = 0; i < n; ++i) {
        float r = nearbyintf(v[i] / s);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        q[i] = (int8_t)r;
    }
    return s;
}

/* Per-row quantization of a row-major [rows, cols] fp32 array. Used for X (per row m)
 * and, on the column-major W stored as [N][K], for W (per output column n). */
void oracle_quant_rows_i8(const float* x, int64_t rows, int64_t cols, int8_t* q, float* scale)
{
    for (int64_t r = 0; r < rows; ++r)
        scale[r] = quant_vec_i8(x + r * cols, cols, q + r * cols);
}

/* Per-tensor symmetric quantization (one scale for the whole array): the
 * baseline that per-channel scales are compared against. */
float oracle_quant_tensor_i8(const float* x, int64_t n, int8_t* q)
{
    return quant_vec_i8(x, n, q);
}

/* ----------------------------------------------- asymmetric int8 (per row) */

/* Asymmetric int8 quantization of each row of a row-major [rows, cols] fp32 array, as the
 * asymmetric branch of hotelren.com's per_channel_quant_int8 computes it, in fp32:
 *   lo, hi = min, max of the row;   s = max((hi - lo) / 255, 1e-8)
 *   z = -lo / s - 128       (kept as a float: the page does not round the zero point)
 *   q = clamp(rne(x / s + z), -128, 127)
 * so that x ~ s (q - z) (quant67.com ch.17 §二, asymmetric form). */
void oracle_quant_rows_i8_asym(const float* x, int64_t rows, int64_t cols, int8_t* q,
                               float* scale, float* zero)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* v = x + r * cols;
        float lo = v[0], hi = v[0];
        for (int64_t i = 1; i < cols; ++i) {
            if (v[i] < lo)
                lo = v[i];
            if (v[i] > hi)
                hi = v[i];
        }
        float s = (hi - lo) / 255.0f;
        if (s < 1e-8f)
            s = 1e-8f;
        const float z = -lo / s - 128.0f;
        for (int64_t i = 0; i < cols; ++i) {
            const float t = v[i] / s + z;
            float rq = nearbyintf(t);
            if (rq > 127.0f)
                rq = 127.0f;
            if (rq < -128.0f)
                rq = -128.0f;
            q[r * cols + i] = (int8_t)rq;
        }
        scale[r] = s;
        zero[r] = z;
    }
}

/* colsum[n] = sum_k wq[n][k]: W's per-column code sums ([N][K] storage). */
void oracle_column_sums_i8(const int8_t* wq, int64_t N, int64_t K, int32_t* colsum)
{
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = 0;
        for (int64_t k = 0; k < K; ++k)
            t += wq[n * K + k];
        colsum[n] = (int32_t)t;
    }
}

/* The layer with asymmetric activations and symmetric per-channel weights, from its
 * definition, in fp64:  y[m][n] = sum_k x_scale[m] (xq[m][k] - x_zero[m]) * w_scale[n] wq[n][k]
 * + bias[n]  (quant67.com ch.17 §二: x ~ s_x (q_x - z_x), w ~ s_w q_w). bias may be NULL. */
void oracle_w8a8_asym_f64(const int8_t* xq, const float* x_scale, const float* x_zero,
                          const int8_t* wq, const float* w_scale, const float* bias, int64_t M,
                          int64_t N, int64_t K, double* y64)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += ((double)xq[m * K + k] - (double)x_zero[m]) * (double)wq[n * K + k];
            double y = acc * (double)x_scale[m] * (double)w_scale[n];
            if (bias)
                y += (double)bias[n];
            y64[m * N + n] = y;
        }
    }
}

/* ------------------------------------------------------------ fp8 (e4m3) */

/* The OCP 8-bit float E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities; the largest
 * finite value is S.1111.110 = 448. */
double oracle_e4m3_decode(uint8_t c)
{
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    const double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* The e4m3 code nearest to x (|x| <= 448), ties to the code with an even mantissa (round
 * half to even), found by search over the finite magnitudes. */
uint8_t oracle_e4m3_encode(float x)
{
    const double a = fabs((double)x);
    int best = 0;
    double bd = a;   /* distance to code 0 */
    for (int c = 1; c < 127; ++c) {   /* 0x7F is NaN */
        const double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* Per-row fp8 quantization (hotelren.com: per_channel_quant_fp8 differs from the int8
 * quantizer only in the result type): s = max(absmax, 1e-10) / 448 (fp32), q = e4m3(x / s)
 * with x / s correctly rounded in fp32, then rounded to e4m3 half to even. */
void oracle_quant_rows_e4m3(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* v = x + r * cols;
        float a = 0.0f;
        for (int64_t i = 0; i < cols; ++i) {
            const float t = fabsf(v[i]);
            if (t > a)
                a = t;
        }
        const float s = (a > 1e-10f ? a : 1e-10f) / 448.0f;
        for (int64_t i = 0; i < cols; ++i) {
            float t = v[i] / s;
            if (t > 448.0f)
                t = 448.0f;
            if (t < -448.0f)
                t = -448.0f;
            q[r * cols + i] = oracle_e4m3_encode(t);
        }
        scale[r] = s;
    }
}

/* The fp8 layer in fp64: y[m][n] = x_scale[m] w_scale[n] sum_k dec(xq[m][k]) dec(wq[n][k])
 * + bias[n]. Also returns mag[m][n] = x_scale w_scale sum_k |dec(xq) dec(wq)| (the scale of
 * an fp32 summation's error) when mag is not NULL. */
void oracle_gemm_e4m3_f64(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                          const float* w_scale, const float* bias, int64_t M, int64_t N,
                          int64_t K, double* y64, double* mag)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, am = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = lut[xq[m * K + k]] * lut[wq[n * K + k]];
                acc += p;
                am += fabs(p);
            }
            const double sc = (double)x_scale[m] * (double)w_scale[n];
            y64[m * N + n] = acc * sc + (bias ? (double)bias[n] : 0.0);
            if (mag)
                mag[m * N + n] = am * sc;
        }
    }
}

/* ---------------------------------------------------------- integer GEMM */

/* acc[m][n] = sum_k xq[m][k] * wq[n][k]; xq is [M][K] row-major, wq is W [K,N]
 * column-major ([N][K] in memory). Returns 0, or 1 if a sum left the int32 range
 * (impossible for codes in [-128, 127] and K < 2^17). */
int oracle_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                    int32_t* acc)
{
    int bad = 0;
#pragma omp parallel for reduction(| : bad) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k)
                t += (int32_t)xq[m * K + k] * (int32_t)wq[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN)
                bad = 1;
            acc[m * N + n] = (int32_t)t;
        }
    }
    return bad;
}

/* y = ((float(acc) * x_scale[m]) * w_scale[n]) + bias[n] in fp32, left to right, and
 * the same quantity in fp64. bias may be NULL (adds nothing). Either output may be NULL. */
void oracle_epilogue_w8a8(const int32_t* acc, const float* x_scale, const float* w_scale,
                          const float* bias, int64_t M, int64_t N, float* y32, double* y64)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t a = acc[m * N + n];
            if (y32) {
                float t = (float)a;
                float y = t * x_scale[m];
                y = y * w_scale[n];
                if (bias)
                    y = y + bias[n];
                y32[m * N + n] = y;
            }
            if (y64) {
                double y = (double)a * (double)x_scale[m] * (double)w_scale[n];
                if (bias)
                    y += (double)bias[n];
                y64[m * N + n] = y;
            }
        }
    }
}

/* ------------------------------------------------ re-quantization of Y */

/* Calibrated static scales of a layer's output, one per output channel (2048ai.net, INT8
 * Llama-2-7B write-up, §3.2-§3.3: the maximum |output| of each channel over the
 * calibration rows, scale = max / 127), with the absmax floor of the other quantizers:
 *   s[n] = max(max_m |y[m][n]|, 1e-10) / 127      (fp32), y row-major [M][N] */
void oracle_channel_scales(const float* y, int64_t M, int64_t N, float* s)
{
    for (int64_t n = 0; n < N; ++n) {
        float a = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            const float t = fabsf(y[m * N + n]);
            if (t > a)
                a = t;
        }
        s[n] = (a > 1e-10f ? a : 1e-10f) / 127.0f;
    }
}

/* Int8 codes of the layer's output with static scales, for a following int8 layer:
 *   q[m][n] = clamp(rne(y[m][n] / s[n]), -127, 127)       (fp32 division)
 * with one scale per output channel (scale_n == N; 2048ai.net §3.2-§3.3) or one for the
 * whole output (scale_n == 1; hotelren.com "量化算法的本质", per_tensor_quant_int8). The code
 * rule is the symmetric quantizers' (quant67.com ch.17 §二). */
void oracle_requant_i8(const float* y, int64_t M, int64_t N, const float* s, int64_t scale_n,
                       int8_t* q)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const float sc = s[scale_n == 1 ? 0 : n];
            float r = nearbyintf(y[m * N + n] / sc);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[m * N + n] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------ weight-only paths */

/* y64[m][n] = sum_k x[m][k] * (q[k][n] - z) * s, in fp64.
 *   codes_kind 0: int8 codes, symmetric (zp must be NULL)
 *   codes_kind 1: uint8 codes with zero points zp
 *   group == 0: one scale per column, scale[n]
 *   group  > 0: scale and zp are [K/group, N] column-major, i.e. [N][K/group]
 * x is fp32 (an fp16 activation converted exactly). codes are [N][K]. */
void oracle_wonly_f64(const float* x, int64_t M, int64_t K, const void* codes, int codes_kind,
                      const float* scale, const uint8_t* zp, int64_t group, const float* bias,
                      int64_t N, double* y64)
{
    const int8_t* q8 = (const int8_t*)codes;
    const uint8_t* u8 = (const uint8_t*)codes;
    int64_t G = group > 0 ? K / group : 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = group > 0 ? k / group : 0;
                double q = codes_kind == 0 ? (double)q8[n * K + k] : (double)u8[n * K + k];
                double z = zp ? (double)zp[n * G + g] : 0.0;
                double s = group > 0 ? (double)scale[n * G + g] : (double)scale[n];
                acc += (double)x[m * K + k] * ((q - z) * s);
            }
            if (bias)
                acc += (double)bias[n];
            y64[m * N + n] = acc;
        }
    }
}

/* The same weight-only product summed in fp32 in k order: w = (q - z) * s rounded to fp32,
 * then acc = RN(acc + RN(x * w)) for k = 0 .. K-1, then + bias. One legitimate fp32 order;
 * its distance from the fp64 value shows how far fp32 summation orders spread at a shape
 * (the tolerance of the weight-only tests must cover any of them). */
void oracle_wonly_f32seq(const float* x, int64_t M, int64_t K, const void* codes, int codes_kind,
                         const float* scale, const uint8_t* zp, int64_t group, const float* bias,
                         int64_t N, float* y32)
{
    const int8_t* q8 = (const int8_t*)codes;
    const uint8_t* u8 = (const uint8_t*)codes;
    int64_t G = group > 0 ? K / group : 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = group > 0 ? k / group : 0;
                float q = codes_kind == 0 ? (float)q8[n * K + k] : (float)u8[n * K + k];
                float z = zp ? (float)zp[n * G + g] : 0.0f;
                float sc = group > 0 ? scale[n * G + g] : scale[n];
                float w = (q - z) * sc;
                float p = x[m * K + k] * w;
                acc = acc + p;
            }
            if (bias)
                acc = acc + bias[n];
            y32[m * N + n] = acc;
        }
    }
}

/* Signed int4 code of element k from column n's packed words ([N][K/8] int32). */
static int unpack_int4(const int32_t* packed, int64_t K, int64_t n, int64_t k)
{
    uint32_t word = (uint32_t)packed[n * (K / 8) + k / 8];
    int nib = (int)((word >> (4 * (k % 8))) & 0xFu);
    return nib >= 8 ? nib - 16 : nib;   /* two's complement */
}

/* y64[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n], in fp64. scale16 holds
 * binary16 bits, [K/group, N] column-major ([N][K/group]). */
void oracle_w4a16_f64(const float* x, int64_t M, int64_t K, const int32_t* packed,
                      const uint16_t* scale16, int64_t group, const float* bias, int64_t N,
                      double* y64)
{
    int64_t G = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double s = (double)oracle_f16_to_f32(scale16[n * G + k / group]);
                acc += (double)x[m * K + k] * ((double)unpack_int4(packed, K, n, k) * s);
            }
            if (bias)
                acc += (double)bias[n];
            y64[m * N + n] = acc;
        }
    }
}

void oracle_unpack_int4(const int32_t* packed, int64_t N, int64_t K, int8_t* q)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = (int8_t)unpack_int4(packed, K, n, k);
}

/* --------------------------------------------------- weight producers */

/* Block-wise asymmetric uint8 quantization of W ([N][K]) in blocks of `block` along K:
 *   mn, mx = min, max over the block; s = max((mx - mn) / 255, 1e-8) (fp32);
 *   zp = clamp(rne(-mn / s), 0, 255); q = clamp(rne(w / s) + zp, 0, 255). */
void oracle_quant_block_asym_u8(const float* w, int64_t N, int64_t K, int64_t block,
                                uint8_t* q, float* scale, uint8_t* zp)
{
    int64_t G = K / block;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* v = w + n * K + g * block;
            float mn = v[0], mx = v[0];
            for (int64_t i = 1; i < block; ++i) {
                if (v[i] < mn)
                    mn = v[i];
                if (v[i] > mx)
                    mx = v[i];
            }
            float s = (mx - mn) / 255.0f;
            if (s < 1e-8f)
                s = 1e-8f;
            float zf = nearbyintf(-mn / s);
            int z = zf < 0.0f ? 0 : (zf > 255.0f ? 255 : (int)zf);
            for (int64_t i = 0; i < block; ++i) {
                int c = (int)nearbyintf(v[i] / s) + z;
                if (c < 0)
                    c = 0;
                if (c > 255)
                    c = 255;
                q[n * K + g * block + i] = (uint8_t)c;
            }
            scale[n * G + g] = s;
            zp[n * G + g] = (uint8_t)z;
        }
    }
}

/* Per-group symmetric int4 quantization of W ([N][K]) in groups of `group` along K:
 *   a = max |w| over the group; s16 = fp16(max(a, 7 * 2^-24) / 7);
 *   q = clamp(rne(w / float(s16)), -8, 7), packed eight per int32 along K. */
void oracle_quant_int4_group(const float* w, int64_t N, int64_t K, int64_t group,
                             int32_t* packed, uint16_t* scale16)
{
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 8; ++j)
            packed[n * (K / 8) + j] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* v = w + n * K + g * group;
            float a = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                float t = fabsf(v[i]);
                if (t > a)
                    a = t;
            }
            const float floor_a = 7.0f * 0x1p-24f;
            uint16_t h = oracle_f32_to_f16((a > floor_a ? a : floor_a) / 7.0f);
            float s = oracle_f16_to_f32(h);
            scale16[n * G + g] = h;
            for (int64_t i = 0; i < group; ++i) {
                float r = nearbyintf(v[i] / s);
                if (r > 7.0f)
                    r = 7.0f;
                if (r < -8.0f)
                    r = -8.0f;
                int64_t k = g * group + i;
                uint32_t nib = (uint32_t)((int)r) & 0xFu;
                uint32_t* word = (uint32_t*)&packed[n * (K / 8) + k / 8];
                *word |= nib << (4 * (k % 8));
            }
        }
    }
}

/* ------------------------------------------------------------ activations */

/* The activation the epilogue applies to the layer's output (after the scales and the
 * bias, before the output is rounded), elementwise and in place, in fp64:
 *   act 1, GELU: y * Phi(y), Phi the standard normal distribution function,
 *          Phi(y) = (1 + erf(y / sqrt 2)) / 2, the exact form (the pages name GELU and
 *          give no approximation)
 *   act 2, SiLU: y * sigmoid(y) = y / (1 + exp(-y))
 *   act 0: none.
 * quant67.com ch.17 §四 (scales, bias and the activation applied in the epilogue while
 * the result is in registers); xdnf.cn INT4/FP16 mixed GEMM §8 (GELU fused after the
 * INT4 GEMM, with no intermediate write-back). */
void oracle_activation_f64(double* y, int64_t n, int act)
{
    for (int64_t i = 0; i < n; ++i) {
        double v = y[i];
        if (act == 1)
            y[i] = v * (0.5 * (1.0 + erf(v / sqrt(2.0))));
        else if (act == 2)
            y[i] = v / (1.0 + exp(-v));
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
