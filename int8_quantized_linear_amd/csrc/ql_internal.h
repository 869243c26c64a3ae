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

// The standard normal tail Phi(-z) for z >= 0, as 2^P(u) with u = min(z / 8, 1): log2 of the
// tail is smooth on [0, 8] (it falls from -1 to about -50), and P is a degree-11 polynomial
// fitted to it with the error allowed at z the smaller of 1e-5 relative and 1e-7 absolute
// (int8_quantized_linear_amd/gelu_tail_fit.py, which also prints this table). In this fp32
// order the GELU below is within 9e-8 |y| of y Phi(y) for every y, within 5e-6 relative for
// y in (-6, 0), and rounds to the correctly rounded fp16 value for all but 3 of the 63,488
// finite fp16 inputs (one fp16 step away for those). Past z = 8 the tail stays at
// Phi(-8) ~ 6.2e-16. Eleven fused multiply-adds and one exp2, no reciprocal and no branch.
__device__ inline float normal_tail(float z) {
    constexpr float c[12] = {7.989465714e+00f, -4.585392761e+01f, 1.142428360e+02f, -1.604418030e+02f,
                             1.351405334e+02f, -6.053829956e+01f, -3.572053194e+00f, 2.901321411e+01f,
                             -2.689651489e+01f, -2.938829422e+01f, -9.208859444e+00f, -9.999999404e-01f};
    const float u = fminf(fmaxf(z * 0.125f, 0.0f), 1.0f);   // one multiply with the clamp modifier
    float p = c[0];
#pragma unroll
    for (int i = 1; i < 12; ++i)
        p = fmaf(p, u, c[i]);
    return __builtin_amdgcn_exp2f(p);
}

// The same tail for epilogues whose output is fp16, where the result only has to land within a
// small fraction of an fp16 step (at least 4.9e-4 of the value): a degree-7 polynomial fitted
// with one relative error bound (gelu_tail_fit.py, fit_f16), within 3.3e-5 of Phi(-z) relative
// on [0, 8]. The GELU below is then within 1.5e-5 |y| of y Phi(y), within 3.2e-5 relative for y
// in (-6, 0), and within one fp16 step of the correctly rounded fp16 value for every finite
// fp16 input. Seven fused multiply-adds instead of eleven.
__device__ inline float normal_tail_f16out(float z) {
    constexpr float c16[8] = {-2.647568226e+00f, 1.263620567e+01f, -2.645191193e+01f, 3.254099274e+01f,
                              -2.694931412e+01f, -2.943723869e+01f, -9.204879761e+00f, -1.000043035e+00f};
    const float u = fminf(fmaxf(z * 0.125f, 0.0f), 1.0f);   // one multiply with the clamp modifier
    float p = c16[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        p = fmaf(p, u, c16[i]);
    return __builtin_amdgcn_exp2f(p);
}

// The epilogue's activation of an fp32 value: GELU in its exact form y * Phi(y), or SiLU
// y * sigmoid(y). GELU is evaluated as max(y, 0) - |y| Phi(-|y|) (equal for every y, since
// y Phi(y) = y - y Phi(-y)), which needs the normal tail only and has no cancellation for
// negative y. F16OUT: the value is rounded to fp16 next, and the shorter tail serves; else
// the error is well below the fp32 epilogue's own.
template <int ACT, bool F16OUT = false>
__device__ inline float activation(float y) {
    if constexpr (ACT == ACT_GELU) {
        const float z = fabsf(y);
        return fmaf(-z, F16OUT ? normal_tail_f16out(z) : normal_tail(z), fmaxf(y, 0.0f));
    } else if constexpr (ACT == ACT_SILU) {
        return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
    } else {
        return y;
    }
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
