/*
 * ql.h -- C ABI of libql.so, a quantized linear layer for AMD Instinct MI355X (gfx950)
 *
 *     Y = (x_scale (.) Xq) @ (w_scale (.) Wq) + bias
 *
 * Sources of the operation (web pages; cited by title and section):
 *   [hotelren]  hotelren.com, "量化算法的本质" -- the statement of Y = XW with X [M,K]
 *               row-major and W [K,N] column-major (opening section); the
 *               per_tensor_quant_int8 and per_channel_quant_int8 quantizers; the list
 *               of a quantized GEMM's parameters (X, W, scale, optional zero, optional
 *               bias) in "量化模型的矩阵乘法"; and Y = (x_scale*X)@(w_scale*W)+bias in
 *               "W8A8矩阵乘法".
 *   [quant67]   quant67.com GPU-kernel series ch.17, "量化与多精度算子：INT8 / FP8、反量化
 *               与 per-channel" -- §二 q = round(x/s) + z and the integer-GEMM expansion;
 *               §三 granularity; §四 int32 accumulation and dequantization in the
 *               epilogue, weight-only dequantization inside the kernel; §六 pitfalls.
 *   [2048ai]    2048ai.net, INT8 Llama-2-7B on Ascend write-up -- §2.2 scale = max/127;
 *               §4 per-output-channel weight scales; §5.2-§5.4 the per-channel INT8 GEMM
 *               C = (A_int8 B_int8) (.) scales[N] with int32 accumulation and dequant at
 *               write-back.
 *   [zingnex]   zingnex.cn, "从零实现大语言模型 INT8 量化" -- 核心量化流程 steps 1-2:
 *               blocks of 64, scale = (max-min)/255, zero_point = round(-min/scale).
 *   [xdnf]      xdnf.cn, INT4/FP16 mixed-precision GEMM as a CANN TBE operator -- §3.2
 *               unpack then dequantize with fp32 accumulation; §4.1 the operator's
 *               (M,K) fp16 x packed int4 -> (M,N) fp16 contract; §5.1 scale = absmax/7.
 *
 * Conventions for every entry point:
 *   - Every array is a DEVICE pointer owned by the caller. The library never
 *     allocates, frees, retains or synchronizes, and keeps no state.
 *   - All work is enqueued on `stream` and the call returns without waiting. Device
 *     faults surface at the caller's next synchronization on that stream. The `stream`
 *     parameter is declared `void*` so that this header needs no HIP include; it is a
 *     hipStream_t (HIP defines that as a pointer to an opaque struct, so the two have
 *     the same size and calling convention). NULL is the null stream.
 *   - Layouts: X and Y are row-major and contiguous. W [K,N] is column-major, i.e. an
 *     [N][K] array with K contiguous ([hotelren] opening section). Per-group scales
 *     and zero points are column-major [K/group, N], i.e. [N][K/group].
 *   - Outputs must not overlap inputs or each other.
 *   - Shapes: M == 0 or N == 0 is an empty problem: QL_OK, nothing is launched.
 *   - All arguments are validated before anything is enqueued; on any error nothing is
 *     written. Validation touches no GPU, so it can be exercised without one.
 *     QL_ERR_NULL  a required pointer is NULL
 *     QL_ERR_SHAPE a size is negative or breaks the divisibility stated per call
 *     QL_ERR_ALIGN a large operand (X, W, Y, codes) is not 16-byte aligned, or a
 *                  scale/bias/zero array is not aligned to its element size (to 4
 *                  bytes for the weight-only calls' scale and zero-point arrays)
 *     QL_ERR_DTYPE an unknown dtype code
 *     QL_ERR_DEVICE the HIP launch reported an error (hipGetLastError)
 *   - Inputs are assumed finite (no NaN or Inf).
 *   - Quantization rounds half to even, divides in correctly rounded fp32 (x / s with
 *     s = absmax / 127, never x * (127 / absmax)) and clamps symmetric codes to
 *     [-127, 127]; an all-zero row or column gets absmax floored at 1e-10.
 */
#ifndef QL_H
#define QL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QL_OK = 0,
    QL_ERR_NULL = 1,
    QL_ERR_SHAPE = 2,
    QL_ERR_ALIGN = 3,
    QL_ERR_DTYPE = 4,
    QL_ERR_DEVICE = 5
} ql_status;

typedef enum { QL_F32 = 0, QL_F16 = 1 } ql_dtype;

/* Activation an epilogue applies to the output after the scales and the bias, in fp32,
 * before the output is rounded: GELU in its exact form y * Phi(y), Phi the standard
 * normal distribution function ((1 + erf(y / sqrt 2)) / 2), or SiLU y / (1 + exp(-y)).
 * [quant67] §四 (scales, bias and activation in the epilogue, while the result is in
 * registers); [xdnf] §8 (GELU fused after the INT4 GEMM, no intermediate write-back).
 * An unknown value is QL_ERR_DTYPE. */
typedef enum { QL_ACT_NONE = 0, QL_ACT_GELU = 1, QL_ACT_SILU = 2 } ql_activation;

/* Human-readable name of a status code (a static string). */
const char* ql_status_str(ql_status s);

/*
 * Per-row (per-token) dynamic symmetric int8 quantization of activations.
 * [hotelren] per_channel_quant_int8 (symmetric branch, absmax along the last
 * dimension, clamp_min 1e-10, scale = absmax/127, torch.round); [2048ai] §2.2.
 *
 *   a[m] = max_k |x[m,k]|,  x_scale[m] = max(a[m], 1e-10) / 127   (fp32)
 *   xq[m,k] = clamp(round_half_even(x[m,k] / x_scale[m]), -127, 127)
 *
 * x       [M,K] row-major, fp32 (x_dtype QL_F32) or fp16 (QL_F16)
 * xq      [M,K] int8 row-major (out)
 * x_scale [M] fp32 (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status quantize_per_row_int8(const void* x, ql_dtype x_dtype, int64_t M, int64_t K,
                                int8_t* xq, float* x_scale, void* stream);

/*
 * Per-tensor symmetric int8 quantization: one scale for the whole array. [hotelren]
 * "量化算法的本质", per_tensor_quant_int8 (global absmax, scale = absmax/127, a scale tensor
 * of one fp32 element); "量化模型的矩阵乘法" (a scale of shape [1] means per-tensor).
 *
 *   a = max_i |x[i]|,  x_scale[0] = max(a, 1e-10) / 127            (fp32)
 *   xq[i] = clamp(round_half_even(x[i] / x_scale[0]), -127, 127)
 *
 * x       n elements, fp32 (QL_F32) or fp16 (QL_F16), contiguous (any shape, flattened)
 * xq      n int8 codes (out);  x_scale one fp32 (out)
 * x_scale also serves as the running maximum while the call's kernels run: it holds its
 * final value once the stream has passed the call. Requires n % 16 == 0.
 */
ql_status quantize_per_tensor_int8(const void* x, ql_dtype x_dtype, int64_t n, int8_t* xq,
                                   float* x_scale, void* stream);

/*
 * Per-output-channel symmetric int8 quantization of weights (offline, before serving).
 * [2048ai] §4.2 and §6.1 (one scale per output channel n); [hotelren]
 * per_channel_quant_int8. Same arithmetic as quantize_per_row_int8, per column n.
 *
 * w       W [K,N] fp32, column-major ([N][K])
 * wq      W [K,N] int8, column-major ([N][K]) (out)
 * w_scale [N] fp32 (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status quantize_weight_per_channel(const float* w, int64_t K, int64_t N, int8_t* wq,
                                      float* w_scale, void* stream);

/*
 * W8A8 GEMM with int32 accumulation and a fused dequantization + bias epilogue.
 * [hotelren] "W8A8矩阵乘法": Y = (x_scale*X) @ (w_scale*W) + bias; [quant67] §四
 * (int32 accumulate, scales and bias applied in the epilogue while in registers);
 * [2048ai] §5.2-§5.4.
 *
 *   acc[m,n] = sum_k xq[m,k] * wq[k,n]          (int32, exact)
 *   y[m,n]   = float(acc) * x_scale[m] * w_scale[n] + bias[n]
 *
 * xq      [M,K] int8 row-major;  x_scale [M] fp32
 * wq      W [K,N] int8 column-major ([N][K]);  w_scale [N] fp32
 * bias    [N] fp32, or NULL for none
 * y       [M,N] row-major, fp32 (y_dtype QL_F32) or fp16 (QL_F16, rounded to nearest even)
 * Requires K > 0, K % 64 == 0 and K <= 131008 (so that |acc| < 2^31 for any codes), and
 * N <= 2^23 (the epilogue addresses 32 output rows with 31-bit byte offsets).
 */
ql_status gemm_w8a8_per_channel(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                const float* w_scale, const float* bias, void* y,
                                ql_dtype y_dtype, int64_t M, int64_t N, int64_t K,
                                void* stream);

/*
 * gemm_w8a8_per_channel with an activation fused into the epilogue:
 *   y[m,n] = act(x_scale[m] * w_scale[n] * acc[m,n] + bias[n])
 * Arguments as for gemm_w8a8_per_channel; act as ql_activation above.
 */
ql_status gemm_w8a8_per_channel_act(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, const float* bias, ql_activation act,
                                    void* y, ql_dtype y_dtype, int64_t M, int64_t N, int64_t K,
                                    void* stream);

/*
 * Asymmetric activations ([hotelren] per_channel_quant_int8, its asymmetric branch;
 * [quant67] §二, x ~ s (q - z) and the expansion of the integer product). Per row m of X,
 * with lo, hi the row's minimum and maximum, in fp32:
 *   s = max((hi - lo) / 255, 1e-8);  z = -lo / s - 128 (kept as a float, as on the page);
 *   q = clamp(round(x / s + z), -128, 127)          (x / s correctly rounded, then + z)
 * x       [M,K] row-major, fp32 (QL_F32) or fp16 (QL_F16)
 * xq      [M,K] int8 row-major (out);  x_scale, x_zero fp32 [M] (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status quantize_per_row_int8_asym(const void* x, ql_dtype x_dtype, int64_t M, int64_t K,
                                     int8_t* xq, float* x_scale, float* x_zero, void* stream);

/*
 * colsum[n] = sum_k wq[k,n]: the per-column code sums of W, the weight-side term of the
 * asymmetric expansion sum_k (q_x - z_x) q_w = sum_k q_x q_w - z_x sum_k q_w ([quant67] §二).
 * An offline step beside the weight quantizer.
 * wq      W [K,N] int8 column-major ([N][K]);  colsum int32 [N] (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status weight_column_sums_i8(const int8_t* wq, int64_t K, int64_t N, int32_t* colsum,
                                void* stream);

/*
 * The layer with asymmetric activations and symmetric per-channel weights:
 *   y[m,n] = act(x_scale[m] * w_scale[n] * (acc[m,n] - x_zero[m] * w_colsum[n]) + bias[n])
 * with acc the exact int32 product of the codes and the correction taken in fp32 with one
 * rounding. Arguments as for gemm_w8a8_per_channel_act, plus x_zero (fp32 [M], from
 * quantize_per_row_int8_asym) and w_colsum (int32 [N], from weight_column_sums_i8).
 */
ql_status gemm_w8a8_asym(const int8_t* xq, const float* x_scale, const float* x_zero,
                         const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                         const float* bias, ql_activation act, void* y, ql_dtype y_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * FP8 (OCP E4M3) variant of the per-row quantizer. [hotelren] "量化算法的本质": the fp8
 * per-channel quantizer is the int8 one with another result type; [quant67] ch.17 (INT8 /
 * FP8). E4M3 (bias 7, 3 mantissa bits, largest finite value 448, S.1111.111 NaN, no
 * infinities) takes the place of [-127, 127]:
 *   x_scale[m] = max(a[m], 1e-10) / 448   (fp32)
 *   xq[m,k]    = e4m3(clamp(x[m,k] / x_scale[m], -448, 448))
 * with x / s correctly rounded in fp32 and e4m3() rounding to nearest, ties to even; a
 * value that rounds to zero keeps its sign (code 0x80 for a negative one).
 * x       [M,K] row-major, fp32 (QL_F32) or fp16 (QL_F16)
 * xq      [M,K] E4M3 codes, one byte each, row-major (out);  x_scale [M] fp32 (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status quantize_per_row_e4m3(const void* x, ql_dtype x_dtype, int64_t M, int64_t K,
                                uint8_t* xq, float* x_scale, void* stream);

/*
 * Per-output-channel E4M3 weights: quantize_per_row_e4m3's arithmetic per column n.
 * w       W [K,N] fp32 column-major ([N][K])
 * wq      W [K,N] E4M3 codes, column-major ([N][K]) (out);  w_scale [N] fp32 (out)
 * Requires K > 0 and K % 16 == 0.
 */
ql_status quantize_weight_per_channel_e4m3(const float* w, int64_t K, int64_t N, uint8_t* wq,
                                           float* w_scale, void* stream);

/*
 * The layer with E4M3 operands ([hotelren] "W8A8矩阵乘法" with fp8 codes; [quant67] §四,
 * scales and bias in the epilogue):
 *   y[m,n] = act(x_scale[m] * w_scale[n] * sum_k dec(xq[m,k]) * dec(wq[k,n]) + bias[n])
 * Precision of the sum (gfx950's fp8 matrix cores, as measured): the products are summed
 * in groups of 8 consecutive k, each product truncated toward zero to a multiple of
 * 2^(E - 13), E the group's largest exponent sum e_x + e_w; group sums are accumulated in
 * fp32. So |y - exact| <= x_scale w_scale sum_g 8 * 2^(E_g - 13) plus fp32 rounding of
 * K/8 + 4 additions -- about 2^-13 relative to the largest products, far below the E4M3
 * codes' own 2^-4 spacing. Arguments, layouts and requirements as for
 * gemm_w8a8_per_channel_act, with one-byte E4M3 codes in place of int8 codes. Codes
 * must not be NaN (0x7F, 0xFF).
 */
ql_status gemm_e4m3_per_channel(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                                const float* w_scale, const float* bias, ql_activation act, void* y,
                                ql_dtype y_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The W8A8 layer with its output re-quantized to int8 for a following int8 layer, in the
 * same epilogue: the result leaves as one byte per element ([quant67] §四: keep bulk data
 * in low precision and convert on chip). The scales are static, as calibrated in [2048ai]
 * §3.2-§3.3 (per output channel, max |output| over calibration rows / 127), or one for
 * the whole output ([hotelren] per_tensor_quant_int8):
 *   y[m,n]  = act(((float(acc[m,n]) * x_scale[m]) * w_scale[n]) + bias[n])
 *             (fp32, each operation rounded on its own, in this order)
 *   yq[m,n] = clamp(round_half_even(y[m,n] / out_scale[n or 0]), -127, 127)
 *             (y / s correctly rounded in fp32)
 * out_scale   fp32, out_scale_n entries: 1 (one scale for all of Y) or N (per column).
 *             Each must be a positive normal fp32 value (a precondition: device memory is
 *             not inspected).
 * yq          [M,N] int8 row-major (out). Other arguments as for gemm_w8a8_per_channel_act.
 * A following W8A8 layer takes yq as its codes with x_scale[m] = out_scale[0] for every row
 * when out_scale_n == 1; per-column scales fold into that layer's weights instead
 * (W'[k,n] = out_scale[k] * W[k,n]).
 * out_scale_n other than 1 or N is QL_ERR_SHAPE.
 */
ql_status gemm_w8a8_requant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, ql_activation act,
                            const float* out_scale, int64_t out_scale_n, int8_t* yq, int64_t M,
                            int64_t N, int64_t K, void* stream);

/*
 * The W8A8 integer accumulators alone, acc[m,n] = sum_k xq[m,k] * wq[k,n] as int32
 * [M,N] row-major. A checking aid for the exact integer stage of
 * gemm_w8a8_per_channel (same main loop); [hotelren] "W8A8矩阵乘法" scheme 1 names
 * this int32 intermediate. Same requirements as gemm_w8a8_per_channel.
 */
ql_status gemm_w8a8_int32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M,
                          int64_t N, int64_t K, void* stream);

/*
 * Weight-only W8A16 GEMM / decode GEMV: fp16 activations, 8-bit weight codes
 * dequantized inside the kernel, fp32 accumulation, fp16 output. [quant67] §四
 * (weight-only: store low-bit weights, dequantize on chip); [hotelren] "量化模型的矩阵
 * 乘法" (optional zero => asymmetric); [zingnex] 核心量化流程 (block-64 uint8).
 *
 *   y[m,n] = sum_k x[m,k] * (q[k,n] - z[g(k),n]) * s[g(k),n] + bias[n]
 *
 * x          [M,K] fp16 row-major
 * wq         W [K,N] column-major ([N][K]): int8 codes if zero_point is NULL, else
 *            uint8 codes
 * w_scale    fp32: [N] if group_size == 0, else [K/group_size, N] column-major
 * zero_point NULL (symmetric), or uint8 with the same shape as w_scale (4-byte aligned)
 * group_size 0 (one scale per output column) or a multiple of 64 dividing K
 * bias       [N] fp32, or NULL
 * y          [M,N] fp16 row-major (out)
 * Requires K > 0, K % 64 == 0 and K <= 2^22.
 */
ql_status gemm_w8a16(const void* x, const void* wq, const float* w_scale,
                     const uint8_t* zero_point, int64_t group_size, const float* bias, void* y,
                     int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Weight-only W4A16 GEMM with per-group symmetric int4 weights. [xdnf] §3.2, §4.1-§4.3
 * (unpack by shift and mask, dequantize, fp16 products with fp32 accumulation, fp16
 * output), §5.1 (scale = absmax/7); [quant67] §三 (per-group scales along K).
 *
 *   y[m,n] = sum_g s[g,n] * sum_{k in g} x[m,k] * q[k,n] + bias[n]
 *
 * x          [M,K] fp16 row-major
 * wq_packed  int32 [N][K/8]: word w of column n holds k = 8w + j in bits [4j, 4j+3],
 *            two's complement (values -8..7)
 * scales     fp16 [K/group_size, N] column-major ([N][K/group_size]), 4-byte aligned
 * group_size a multiple of 64 dividing K
 * bias       [N] fp32, or NULL
 * y          [M,N] fp16 row-major (out)
 * Requires K > 0, K % 64 == 0 and K <= 2^22.
 */
ql_status gemm_w4a16_grouped(const void* x, const int32_t* wq_packed, const void* scales,
                             int64_t group_size, const float* bias, void* y, int64_t M,
                             int64_t N, int64_t K, void* stream);

/*
 * gemm_w4a16_grouped with an activation fused into the epilogue ([xdnf] §8):
 *   y[m,n] = act(sum_g s[g,n] * sum_{k in g} x[m,k] * q[k,n] + bias[n])
 * Arguments as for gemm_w4a16_grouped; act as ql_activation above.
 */
ql_status gemm_w4a16_grouped_act(const void* x, const int32_t* wq_packed, const void* scales,
                                 int64_t group_size, const float* bias, ql_activation act, void* y,
                                 int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Producer of the block-asymmetric uint8 weight format consumed by gemm_w8a16.
 * [zingnex] 核心量化流程 steps 1-2, per block b of `block` weights along K and column n:
 *   s = max((max - min) / 255, 1e-8) (fp32);  zp = clamp(round(-min / s), 0, 255)
 *   q = clamp(round(w / s) + zp, 0, 255)                       (round half to even)
 *
 * w          W [K,N] fp32 column-major ([N][K])
 * wq         uint8 [N][K] (out);  scale fp32 [N][K/block] (out);  zero_point uint8
 *            [N][K/block] (out)
 * Requires K > 0, block % 16 == 0, K % block == 0.
 */
ql_status quantize_weight_block_asym_u8(const float* w, int64_t K, int64_t N, int64_t block,
                                        uint8_t* wq, float* scale, uint8_t* zero_point,
                                        void* stream);

/*
 * Producer of the per-group int4 weight format consumed by gemm_w4a16_grouped.
 * [xdnf] §5.1, per group g of `group` weights along K and column n:
 *   s16 = fp16(max(absmax, 7 * 2^-24) / 7);  q = clamp(round(w / s16), -8, 7)
 * (codes are taken with the stored fp16 scale; the floor keeps s16 > 0).
 *
 * w          W [K,N] fp32 column-major ([N][K])
 * wq_packed  int32 [N][K/8] (out), layout as in gemm_w4a16_grouped
 * scales     fp16 [N][K/group] (out)
 * Requires K > 0, group % 16 == 0, K % group == 0.
 */
ql_status quantize_weight_int4_grouped(const float* w, int64_t K, int64_t N, int64_t group,
                                       int32_t* wq_packed, void* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QL_H */
