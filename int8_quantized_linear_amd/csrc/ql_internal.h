// ql_internal.h -- shared definitions of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ql.h"

namespace ql {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// y = ((t * xs) * ws) + b with every operation rounded on its own (no fused multiply-add),
// the order in which the int8 output's codes are defined.
__device__ inline float epilogue_unfused(float t, float xs, float ws, float b) {
#pragma clang fp contract(off)
    return (t * xs) * ws + b;
}

// int8 code of y with output scale s and r = RN(1 / s): the correctly rounded quotient y / s
// as q0 = RN(y r), RN(q0 + fma(-q0, s, y) r), then RNE and the [-127, 127] clamp.
__device__ inline int8_t requant_code(float y, float s, float r) {
    const float q0 = y * r;
    const float qt = fmaf(fmaf(-q0, s, y), r, q0);
    return (int8_t)__builtin_amdgcn_fmed3f(rintf(qt), -127.0f, 127.0f);
}

// Compute units of the current device (256 on MI355X; 256 if the query fails), read once
// per device under std::call_once, so concurrent first calls from several host threads are
// safe. Launch shapes use it to size grids.
constexpr int kMaxDevices = 64;
inline int cu_count() {
    static std::once_flag once[kMaxDevices];
    static int count[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    std::call_once(once[dev], [dev] {
        int v = 0;
        count[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
                         ? v
                         : 256;
    });
    return count[dev];
}

// Launch helpers, one per kernel family. Arguments are already validated; each returns
// QL_OK or QL_ERR_DEVICE (from hipGetLastError after the launch).
ql_status launch_quant_rows_i8(const void* x, int x_is_f16, int64_t rows, int64_t K, int8_t* q,
                               float* scale, hipStream_t stream);
ql_status launch_quant_tensor_i8(const void* x, int x_is_f16, int64_t n, int8_t* q, float* scale,
                                 hipStream_t stream);
ql_status launch_quant_rows_e4m3(const void* x, int x_is_f16, int64_t rows, int64_t K, uint8_t* q,
                                 float* scale, hipStream_t stream);
ql_status launch_quant_rows_i8_asym(const void* x, int x_is_f16, int64_t rows, int64_t K, int8_t* q,
                                    float* scale, float* zero, hipStream_t stream);
ql_status launch_column_sums_i8(const int8_t* wq, int64_t K, int64_t N, int32_t* colsum,
                                hipStream_t stream);
ql_status launch_quant_block_asym_u8(const float* w, int64_t K, int64_t N, int64_t block,
                                     uint8_t* q, float* scale, uint8_t* zp, hipStream_t stream);
ql_status launch_quant_int4_group(const float* w, int64_t K, int64_t N, int64_t group,
                                  int32_t* packed, void* scales, hipStream_t stream);
// x_zero (per row) and colsum (W's column code sums) are NULL for symmetric activations.
// e4m3: xq and wq hold OCP E4M3 fp8 codes (fp32 accumulation; y_mode F32 or F16 only).
// Y_I8: int8 codes clamp(rne(y / out_scale), -127, 127) with out_scale_n = 1 or N scales
// (symmetric activations only).
ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode, int act,
                           const float* x_zero, const int32_t* colsum, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream, bool e4m3 = false,
                           const float* out_scale = nullptr, int out_scale_n = 0);
// The W8A8 layer for M <= 128: y_mode F32, F16 (with zero points when x_zero and colsum are
// given), I32, or I8 (out_scale_n = 1 or N output scales); e4m3: E4M3 codes, F32 or F16 only.
ql_status launch_gemm_w8a8_small(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                 const float* w_scale, const float* bias, void* y, int y_mode, int act,
                                 const float* x_zero, const int32_t* colsum, const float* out_scale,
                                 int out_scale_n, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                                 bool e4m3 = false);
// The W8A8 layer on 64 x 64 tiles (row counts between the few-row kernel's and where the tile
// kernel fills the chip), with the same epilogue modes as launch_gemm_w8a8_small.
ql_status launch_gemm_w8a8_mid(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const float* bias, void* y, int y_mode, int act,
                               const float* x_zero, const int32_t* colsum, const float* out_scale,
                               int out_scale_n, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                               bool e4m3 = false);
ql_status launch_wonly(const void* x, const void* codes, int fmt, const void* scale,
                       const uint8_t* zp, int64_t group, const float* bias, void* y, int64_t M,
                       int64_t N, int64_t K, int act, hipStream_t stream);

// y_mode of launch_gemm_w8a8
enum { Y_F32 = 0, Y_F16 = 1, Y_I32 = 2, Y_I8 = 3 };
// activation applied by an epilogue (values of ql_activation)
enum { ACT_NONE = 0, ACT_GELU = 1, ACT_SILU = 2 };

// erfc(x) for all x from the Chebyshev fit of Numerical Recipes (Press et al., 2nd ed.,
// §6.2, "erfcc"): with z = |x| and t = 1 / (1 + z / 2),
//   erfc(z) ~ t exp(-z^2 - 1.26551223 + t P(t)),   P a degree-8 polynomial,
// fractional error below 1.2e-7 for every z >= 0; erfc(-z) = 2 - erfc(z). One
// reciprocal, nine fused multiply-adds and one exponential, with no range branches (the
// library's erfc branches by range, and lanes of a wave then run several ranges).
__device__ inline float erfc_fit(float x) {
    const float z = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    const float r = t * __expf(fmaf(-z, z, fmaf(t, p, -1.26551223f)));
    return x >= 0.0f ? r : 2.0f - r;
}

// The epilogue's activation of an fp32 value: GELU in its exact form y * Phi(y), or SiLU
// y * sigmoid(y). Phi(y) = erfc(-y / sqrt 2) / 2, the same function as
// (1 + erf(y / sqrt 2)) / 2 without its cancellation for negative y (near -5 the sum
// keeps only a few bits of Phi in fp32). Relative error a few 1e-6 at most: below the
// fp32 epilogue's own for the values that matter, and far below an fp16 step.
template <int ACT>
__device__ inline float activation(float y) {
    if constexpr (ACT == ACT_GELU)
        return 0.5f * y * erfc_fit(-y * 0.70710678118654752f);
    else if constexpr (ACT == ACT_SILU)
        return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
    else
        return y;
}
// fmt of launch_wonly
enum { W_INT8_SYM = 0, W_UINT8_ZP = 1, W_INT4_SYM = 2 };

inline ql_status launch_status() {
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_DEVICE;
}

// Maps a linear workgroup id to a tile id so that, with workgroups dealt round-robin to
// the 8 XCDs, each XCD receives a contiguous run of tile ids (neighbouring tiles share
// operand panels in that XCD's L2).
__device__ inline int xcd_remap(int bid, int ntiles) {
    const int q = ntiles >> 3, r = ntiles & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace ql
