// ql_internal.h -- shared definitions of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ql.h"

namespace ql {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Launch helpers, one per kernel family. Arguments are already validated; each returns
// QL_OK or QL_ERR_DEVICE (from hipGetLastError after the launch).
ql_status launch_quant_rows_i8(const void* x, int x_is_f16, int64_t rows, int64_t K, int8_t* q,
                               float* scale, hipStream_t stream);
ql_status launch_quant_block_asym_u8(const float* w, int64_t K, int64_t N, int64_t block,
                                     uint8_t* q, float* scale, uint8_t* zp, hipStream_t stream);
ql_status launch_quant_int4_group(const float* w, int64_t K, int64_t N, int64_t group,
                                  int32_t* packed, void* scales, hipStream_t stream);
ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);
ql_status launch_wonly(const void* x, const void* codes, int fmt, const void* scale,
                       const uint8_t* zp, int64_t group, const float* bias, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream);

// y_mode of launch_gemm_w8a8
enum { Y_F32 = 0, Y_F16 = 1, Y_I32 = 2 };
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
