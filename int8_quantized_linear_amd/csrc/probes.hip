// probes.hip -- measurement probes for the benchmark (libqlprobe.so), not part of the
// layer: the ceilings that the layer's kernels are compared against on the GPU at hand.
//
// qlp_mfma_i8: every wave issues back-to-back v_mfma_i32_32x32x32_i8 on four independent
// accumulators from registers only, so nothing but the matrix cores limits it. The
// operands are random bytes or one constant pattern: the chip lowers its clock to stay
// within its power limit, and MFMA power depends on the operand bits.
//
// qlp_mfma_i8_data: the same loop on operands loaded once from two code arrays (a layer's
// own quantized W and X), W's as the first operand as in the GEMM: the matrix cores'
// ceiling for that data.
//
// qlp_stream_read: reads a buffer once, 16 bytes a lane with 4 loads in flight per lane on
// one workgroup of 8 waves per CU, and folds the words so that the loads stay live: the rate
// one launch can pull a buffer of a given size out of HBM. That shape was the fastest or
// within 3% of it at every size from 16 MiB to 1 GiB among 4, 8 or 16 waves per workgroup,
// 1, 2 or 4 workgroups per CU and 4, 8 or 16 loads per lane (event-timed bursts); deeper
// queues on fewer waves lose at small sizes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/ql_probe.h"

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;

__device__ inline uint32_t hash32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(THREADS) void mfma_i8_kernel(int64_t iters, int random_operands,
                                                           int32_t* __restrict__ sink) {
    const uint32_t id = blockIdx.x * THREADS + threadIdx.x;
    i32x4 a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[q][e] = random_operands ? (int32_t)hash32(id * 32u + q * 4 + e) : 0x01010101;
            b[q][e] = random_operands ? (int32_t)hash32(id * 32u + 16 + q * 4 + e + 0x9e3779b9u) : 0x01010101;
        }
    i32x16 acc[4] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[q], b[(q + j) & 3], acc[j], 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    sink[id] = s;
}

// Lane t of the grid takes its four 16-byte fragments of each operand from consecutive
// 16-byte pieces at piece 4 t of the array (wrapping around its end): 16 consecutive codes
// of a row, as a fragment holds them.
__global__ __launch_bounds__(THREADS) void mfma_i8_data_kernel(int64_t iters, const i32x4* __restrict__ w,
                                                                int64_t nw16, const i32x4* __restrict__ x,
                                                                int64_t nx16, int32_t* __restrict__ sink) {
    const uint32_t id = blockIdx.x * THREADS + threadIdx.x;
    i32x4 a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a[q] = w[(4 * (int64_t)id + q) % nw16];
        b[q] = x[(4 * (int64_t)id + q) % nx16];
    }
    i32x16 acc[4] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[q], b[(q + j) & 3], acc[j], 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    sink[id] = s;
}

constexpr int READ_THREADS = 512;   // threads per stream-read workgroup (one per CU)
constexpr int READ_DEPTH = 4;       // loads in flight per lane

__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const int64_t nthr = (int64_t)gridDim.x * READ_THREADS;
    const int64_t tid = (int64_t)blockIdx.x * READ_THREADS + threadIdx.x;
    u32x4 f{0, 0, 0, 0};
    for (int64_t base = tid; base < n16; base += READ_DEPTH * nthr) {
        u32x4 r[READ_DEPTH];
#pragma unroll
        for (int t = 0; t < READ_DEPTH; ++t) {
            const int64_t i = base + t * nthr;
            r[t] = i < n16 ? src[i] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < READ_DEPTH; ++t)
            f ^= r[t];
    }
    sink[tid] = f[0] ^ f[1] ^ f[2] ^ f[3];
}

}  // namespace

extern "C" int qlp_cu_count(void) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        return -1;
    return v;
}

extern "C" int qlp_mfma_i8(int64_t iters, int random_operands, int32_t* sink, void* stream) {
    const int cus = qlp_cu_count();
    if (cus <= 0 || sink == nullptr || iters < 0)
        return -1;
    hipLaunchKernelGGL(mfma_i8_kernel, dim3((unsigned)cus), dim3(THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), iters, random_operands, sink);
    return (int)hipGetLastError();
}

extern "C" int qlp_mfma_i8_data(int64_t iters, const int8_t* w, int64_t w_bytes, const int8_t* x,
                                int64_t x_bytes, int32_t* sink, void* stream) {
    const int cus = qlp_cu_count();
    if (cus <= 0 || sink == nullptr || iters < 0 || w == nullptr || x == nullptr || w_bytes < 16 ||
        x_bytes < 16 || w_bytes % 16 != 0 || x_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(w) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(x) % 16 != 0)
        return -1;
    hipLaunchKernelGGL(mfma_i8_data_kernel, dim3((unsigned)cus), dim3(THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), iters, reinterpret_cast<const i32x4*>(w),
                       w_bytes / 16, reinterpret_cast<const i32x4*>(x), x_bytes / 16, sink);
    return (int)hipGetLastError();
}

extern "C" int qlp_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    const int cus = qlp_cu_count();
    if (cus <= 0 || src == nullptr || sink == nullptr || bytes < 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)cus), dim3(READ_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(src),
                       bytes / 16, sink);
    return (int)hipGetLastError();
}
