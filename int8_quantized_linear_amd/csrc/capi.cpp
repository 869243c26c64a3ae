// capi.cpp -- the extern "C" entry points of libql.so: argument validation, then one
// kernel launch on the caller's stream. Validation makes no HIP call, so every error
// path can be exercised on a machine without a GPU. Contracts are stated in ql.h.
#include <stdint.h>

#include "ql_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // sizes are passed to kernels as int
constexpr int64_t kMaxKw8a8 = 131008;           // K * 128^2 < 2^31, K % 64 == 0
constexpr int64_t kMaxNw8a8 = (int64_t)1 << 23; // 32 output rows of 4-byte values: 2^30 bytes
constexpr int64_t kMaxKwonly = (int64_t)1 << 22; // 64 rows of fp16 X and 64 weight columns < 2^31 bytes

// Three W8A8 kernels share the calls: the few-row kernel (gemm_w8a8_small.hip, N / 16
// workgroups each reading all of X), the 64 x 64 tile kernel (gemm_w8a8_mid.hip) and the
// 256 x 256 / 128 x 256 tile kernel (gemm_w8a8.hip); launch_gemm_w8a8 chooses between the
// last two. The few-row kernel's time grows with M * N, the 64 x 64 kernel's stays flat while
// its tiles make one round (M <= 64 up to N = 16384). Measured (us, few-row / 64 x 64) at
// K = 4096: N = 4096 M = 64 11.6 / 12.8, M = 96 14.9 / 13.2; N = 11008 M = 16 14.5 / 16.5,
// M = 32 21.2 / 16.7; N = 14336 M = 1 13.1 / 17.0, M = 16 17.7 / 17.1. The crossover moves
// with N, hardly with K (K = 11008 and 14336 give the same choices within 5%, except
// N = 4096, M = 96 at K = 14336: 41.7 / 43.8).
constexpr int64_t kSmallM = 128;
inline bool few_rows(int64_t M, int64_t N) {
    return M <= kSmallM && (M <= 8 || (M * N <= 256 * 1024 && N <= 12288));
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline bool bad_dims(int64_t M, int64_t N, int64_t K) {
    return M < 0 || N < 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim ||
           M * K >= kMaxDim * 64 || N * K >= kMaxDim * 64 || M * N >= kMaxDim * 64;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* ql_status_str(ql_status s) {
    switch (s) {
    case QL_OK:
        return "QL_OK";
    case QL_ERR_NULL:
        return "QL_ERR_NULL: a required pointer is NULL";
    case QL_ERR_SHAPE:
        return "QL_ERR_SHAPE: a size is negative or breaks the required divisibility";
    case QL_ERR_ALIGN:
        return "QL_ERR_ALIGN: a pointer is not suitably aligned";
    case QL_ERR_DTYPE:
        return "QL_ERR_DTYPE: unknown dtype";
    case QL_ERR_DEVICE:
        return "QL_ERR_DEVICE: the HIP launch failed";
    }
    return "unknown ql_status";
}

ql_status quantize_per_row_int8(const void* x, ql_dtype x_dtype, int64_t M, int64_t K, int8_t* xq,
                                float* x_scale, void* stream) {
    if (x_dtype != QL_F32 && x_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (bad_dims(M, 1, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (M == 0)
        return QL_OK;
    if (!x || !xq || !x_scale)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_rows_i8(x, x_dtype == QL_F16, M, K, xq, x_scale, as_stream(stream));
}

ql_status quantize_per_tensor_int8(const void* x, ql_dtype x_dtype, int64_t n, int8_t* xq,
                                  float* x_scale, void* stream) {
    if (x_dtype != QL_F32 && x_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (n < 0 || n >= kMaxDim * 64 || n % 16 != 0)
        return QL_ERR_SHAPE;
    if (n == 0)
        return QL_OK;
    if (!x || !xq || !x_scale)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_tensor_i8(x, x_dtype == QL_F16, n, xq, x_scale, as_stream(stream));
}

ql_status quantize_weight_per_channel(const float* w, int64_t K, int64_t N, int8_t* wq,
                                      float* w_scale, void* stream) {
    if (bad_dims(1, N, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (N == 0)
        return QL_OK;
    if (!w || !wq || !w_scale)
        return QL_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(w_scale, 4))
        return QL_ERR_ALIGN;
    // Column n of the column-major W is row n of an [N][K] array: the per-row kernel.
    return ql::launch_quant_rows_i8(w, 0, N, K, wq, w_scale, as_stream(stream));
}

static ql_status check_w8a8(const int8_t* xq, const int8_t* wq, const void* y, int64_t M,
                            int64_t N, int64_t K) {
    if (bad_dims(M, N, K) || K % 64 != 0 || K > kMaxKw8a8 || N > kMaxNw8a8)
        return QL_ERR_SHAPE;
    if (M == 0 || N == 0)
        return QL_OK;
    if (!xq || !wq || !y)
        return QL_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16))
        return QL_ERR_ALIGN;
    return QL_OK;
}

ql_status quantize_per_row_int8_asym(const void* x, ql_dtype x_dtype, int64_t M, int64_t K,
                                     int8_t* xq, float* x_scale, float* x_zero, void* stream) {
    if (x_dtype != QL_F32 && x_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (bad_dims(M, 1, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (M == 0)
        return QL_OK;
    if (!x || !xq || !x_scale || !x_zero)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_zero, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_rows_i8_asym(x, x_dtype == QL_F16, M, K, xq, x_scale, x_zero,
                                         as_stream(stream));
}

ql_status weight_column_sums_i8(const int8_t* wq, int64_t K, int64_t N, int32_t* colsum,
                                void* stream) {
    if (bad_dims(1, N, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (N == 0)
        return QL_OK;
    if (!wq || !colsum)
        return QL_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(colsum, 4))
        return QL_ERR_ALIGN;
    return ql::launch_column_sums_i8(wq, K, N, colsum, as_stream(stream));
}

ql_status gemm_w8a8_asym(const int8_t* xq, const float* x_scale, const float* x_zero,
                         const int8_t* wq, const float* w_scale, const int32_t* w_colsum,
                         const float* bias, ql_activation act, void* y, ql_dtype y_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream) {
    if (y_dtype != QL_F32 && y_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (act != QL_ACT_NONE && act != QL_ACT_GELU && act != QL_ACT_SILU)
        return QL_ERR_DTYPE;
    ql_status st = check_w8a8(xq, wq, y, M, N, K);
    if (st != QL_OK || M == 0 || N == 0)
        return st;
    if (!x_scale || !x_zero || !w_scale || !w_colsum)
        return QL_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(x_zero, 4) || !aligned(w_scale, 4) || !aligned(w_colsum, 4) ||
        (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    if (few_rows(M, N))
        return ql::launch_gemm_w8a8_small(xq, x_scale, wq, w_scale, bias, y,
                                          y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, x_zero,
                                          w_colsum, nullptr, 0, M, N, K, as_stream(stream));
    return ql::launch_gemm_w8a8(xq, x_scale, wq, w_scale, bias, y,
                                y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, x_zero, w_colsum,
                                M, N, K, as_stream(stream));
}

ql_status gemm_w8a8_per_channel_act(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, const float* bias, ql_activation act,
                                    void* y, ql_dtype y_dtype, int64_t M, int64_t N, int64_t K,
                                    void* stream) {
    if (y_dtype != QL_F32 && y_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (act != QL_ACT_NONE && act != QL_ACT_GELU && act != QL_ACT_SILU)
        return QL_ERR_DTYPE;
    ql_status st = check_w8a8(xq, wq, y, M, N, K);
    if (st != QL_OK || M == 0 || N == 0)
        return st;
    if (!x_scale || !w_scale)
        return QL_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    if (few_rows(M, N))
        return ql::launch_gemm_w8a8_small(xq, x_scale, wq, w_scale, bias, y,
                                          y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, nullptr,
                                          nullptr, nullptr, 0, M, N, K, as_stream(stream));
    return ql::launch_gemm_w8a8(xq, x_scale, wq, w_scale, bias, y,
                                y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, nullptr, nullptr, M, N, K,
                                as_stream(stream));
}

ql_status quantize_per_row_e4m3(const void* x, ql_dtype x_dtype, int64_t M, int64_t K, uint8_t* xq,
                               float* x_scale, void* stream) {
    if (x_dtype != QL_F32 && x_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (bad_dims(M, 1, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (M == 0)
        return QL_OK;
    if (!x || !xq || !x_scale)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_rows_e4m3(x, x_dtype == QL_F16, M, K, xq, x_scale, as_stream(stream));
}

ql_status quantize_weight_per_channel_e4m3(const float* w, int64_t K, int64_t N, uint8_t* wq,
                                           float* w_scale, void* stream) {
    if (bad_dims(1, N, K) || K % 16 != 0)
        return QL_ERR_SHAPE;
    if (N == 0)
        return QL_OK;
    if (!w || !wq || !w_scale)
        return QL_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(w_scale, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_rows_e4m3(w, 0, N, K, wq, w_scale, as_stream(stream));
}

ql_status gemm_e4m3_per_channel(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                                const float* w_scale, const float* bias, ql_activation act, void* y,
                                ql_dtype y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    if (y_dtype != QL_F32 && y_dtype != QL_F16)
        return QL_ERR_DTYPE;
    if (act != QL_ACT_NONE && act != QL_ACT_GELU && act != QL_ACT_SILU)
        return QL_ERR_DTYPE;
    const int8_t* xc = reinterpret_cast<const int8_t*>(xq);
    const int8_t* wc = reinterpret_cast<const int8_t*>(wq);
    ql_status st = check_w8a8(xc, wc, y, M, N, K);
    if (st != QL_OK || M == 0 || N == 0)
        return st;
    if (!x_scale || !w_scale)
        return QL_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    if (few_rows(M, N))
        return ql::launch_gemm_w8a8_small(xc, x_scale, wc, w_scale, bias, y,
                                          y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, nullptr,
                                          nullptr, nullptr, 0, M, N, K, as_stream(stream), true);
    return ql::launch_gemm_w8a8(xc, x_scale, wc, w_scale, bias, y,
                                y_dtype == QL_F32 ? ql::Y_F32 : ql::Y_F16, (int)act, nullptr, nullptr, M, N, K,
                                as_stream(stream), true);
}

ql_status gemm_w8a8_requant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, ql_activation act,
                            const float* out_scale, int64_t out_scale_n, int8_t* yq, int64_t M,
                            int64_t N, int64_t K, void* stream) {
    if (act != QL_ACT_NONE && act != QL_ACT_GELU && act != QL_ACT_SILU)
        return QL_ERR_DTYPE;
    ql_status st = check_w8a8(xq, wq, yq, M, N, K);
    if (st != QL_OK)
        return st;
    if (out_scale_n != 1 && out_scale_n != N)
        return QL_ERR_SHAPE;
    if (M == 0 || N == 0)
        return QL_OK;
    if (!x_scale || !w_scale || !out_scale)
        return QL_ERR_NULL;
    if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(out_scale, 4) ||
        (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    if (few_rows(M, N))
        return ql::launch_gemm_w8a8_small(xq, x_scale, wq, w_scale, bias, yq, ql::Y_I8, (int)act, nullptr,
                                          nullptr, out_scale, (int)out_scale_n, M, N, K, as_stream(stream));
    return ql::launch_gemm_w8a8(xq, x_scale, wq, w_scale, bias, yq, ql::Y_I8, (int)act, nullptr,
                                nullptr, M, N, K, as_stream(stream), false, out_scale,
                                (int)out_scale_n);
}

ql_status gemm_w8a8_per_channel(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                const float* w_scale, const float* bias, void* y,
                                ql_dtype y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_w8a8_per_channel_act(xq, x_scale, wq, w_scale, bias, QL_ACT_NONE, y, y_dtype, M, N,
                                     K, stream);
}

ql_status gemm_w8a8_int32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M, int64_t N,
                          int64_t K, void* stream) {
    ql_status st = check_w8a8(xq, wq, acc, M, N, K);
    if (st != QL_OK || M == 0 || N == 0)
        return st;
    if (few_rows(M, N))
        return ql::launch_gemm_w8a8_small(xq, nullptr, wq, nullptr, nullptr, acc, ql::Y_I32, ql::ACT_NONE,
                                          nullptr, nullptr, nullptr, 0, M, N, K, as_stream(stream));
    return ql::launch_gemm_w8a8(xq, nullptr, wq, nullptr, nullptr, acc, ql::Y_I32, ql::ACT_NONE, nullptr,
                                nullptr, M, N, K, as_stream(stream));
}

ql_status gemm_w8a16(const void* x, const void* wq, const float* w_scale,
                     const uint8_t* zero_point, int64_t group_size, const float* bias, void* y,
                     int64_t M, int64_t N, int64_t K, void* stream) {
    if (bad_dims(M, N, K) || K % 64 != 0 || K > kMaxKwonly || group_size < 0 ||
        (group_size > 0 && (group_size % 64 != 0 || K % group_size != 0)))
        return QL_ERR_SHAPE;
    if (M == 0 || N == 0)
        return QL_OK;
    if (!x || !wq || !w_scale || !y)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(w_scale, 4) ||
        (zero_point && !aligned(zero_point, 4)) || (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    return ql::launch_wonly(x, wq, zero_point ? ql::W_UINT8_ZP : ql::W_INT8_SYM, w_scale,
                            zero_point, group_size, bias, y, M, N, K, ql::ACT_NONE, as_stream(stream));
}

ql_status gemm_w4a16_grouped_act(const void* x, const int32_t* wq_packed, const void* scales,
                                 int64_t group_size, const float* bias, ql_activation act, void* y,
                                 int64_t M, int64_t N, int64_t K, void* stream) {
    if (act != QL_ACT_NONE && act != QL_ACT_GELU && act != QL_ACT_SILU)
        return QL_ERR_DTYPE;
    if (bad_dims(M, N, K) || K % 64 != 0 || K > kMaxKwonly || group_size <= 0 || group_size % 64 != 0 ||
        K % group_size != 0)
        return QL_ERR_SHAPE;
    if (M == 0 || N == 0)
        return QL_OK;
    if (!x || !wq_packed || !scales || !y)
        return QL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq_packed, 16) || !aligned(y, 16) || !aligned(scales, 4) ||
        (bias && !aligned(bias, 4)))
        return QL_ERR_ALIGN;
    return ql::launch_wonly(x, wq_packed, ql::W_INT4_SYM, scales, nullptr, group_size, bias, y, M,
                            N, K, (int)act, as_stream(stream));
}

ql_status gemm_w4a16_grouped(const void* x, const int32_t* wq_packed, const void* scales,
                             int64_t group_size, const float* bias, void* y, int64_t M, int64_t N,
                             int64_t K, void* stream) {
    return gemm_w4a16_grouped_act(x, wq_packed, scales, group_size, bias, QL_ACT_NONE, y, M, N, K,
                                  stream);
}

ql_status quantize_weight_block_asym_u8(const float* w, int64_t K, int64_t N, int64_t block,
                                        uint8_t* wq, float* scale, uint8_t* zero_point,
                                        void* stream) {
    if (bad_dims(1, N, K) || block <= 0 || block % 16 != 0 || K % block != 0)
        return QL_ERR_SHAPE;
    if (N == 0)
        return QL_OK;
    if (!w || !wq || !scale || !zero_point)
        return QL_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(scale, 4))
        return QL_ERR_ALIGN;
    return ql::launch_quant_block_asym_u8(w, K, N, block, wq, scale, zero_point,
                                          as_stream(stream));
}

ql_status quantize_weight_int4_grouped(const float* w, int64_t K, int64_t N, int64_t group,
                                       int32_t* wq_packed, void* scales, void* stream) {
    if (bad_dims(1, N, K) || group <= 0 || group % 16 != 0 || K % group != 0)
        return QL_ERR_SHAPE;
    if (N == 0)
        return QL_OK;
    if (!w || !wq_packed || !scales)
        return QL_ERR_NULL;
    if (!aligned(w, 16) || !aligned(wq_packed, 16) || !aligned(scales, 2))
        return QL_ERR_ALIGN;
    return ql::launch_quant_int4_group(w, K, N, group, wq_packed, scales, as_stream(stream));
}

}  // extern "C"
