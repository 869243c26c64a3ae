// gemm_w8a8.hip -- W8A8 GEMM on gfx950 int8 MFMA with int32 accumulation and a fused
// dequantization + bias epilogue.
//
//   acc[m,n] = sum_k xq[m,k] * wq[k,n]                 (int32, exact)
//   y[m,n]   = float(acc) * x_scale[m] * w_scale[n] + bias[n]
//
// hotelren.com "量化算法的本质", "W8A8矩阵乘法": Y = (x_scale*X) @ (w_scale*W) + bias with
// X [M,K] row-major int8 and W [K,N] column-major int8, i.e. both operands K-contiguous.
// quant67.com ch.17 §四: int32 accumulators, scales and bias applied in the epilogue
// while the tile is still in registers (no int32 round trip through memory).
// 2048ai.net INT8 Llama-2-7B write-up §5.3: the K loop double-buffers tiles in on-chip
// memory; here that is LDS, filled while the matrix cores work on the other buffer.
//
// Tile: 256 (M) x 256 (N) x 128 (K bytes) per workgroup of 4 waves (2 x 2); each wave
// owns a 128 x 128 block of accumulators = 8 x 8 v_mfma_i32_16x16x64_i8 tiles (256
// accumulator registers per lane). A and B tiles are staged in LDS as rows of 128 bytes
// split in eight 16-byte chunks, XOR-swizzled per row so that the 16 rows a fragment
// read touches fall in distinct bank groups.
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTHR = 256;
constexpr int WM = 128, WN = 128;
constexpr int FM = WM / 16, FN = WN / 16;
constexpr int STAGE = (BM + BN) * BK;      // bytes per LDS stage (A then B)
constexpr int LOADS = BM * BK / 16 / NTHR;  // 16-byte chunks per thread per operand per stage

// Byte offset of 16-byte chunk c (0..7) of tile row r. The chunk index is XORed with a
// row hash that differs across any 8 consecutive rows and across rows r and r + 8.
__device__ inline int swz(int r, int c) {
    return r * BK + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4);
}

template <int YMODE>
__global__ __launch_bounds__(NTHR, 1) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int K, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * STAGE];

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m, tm = tile - tn * tiles_m;  // neighbours share the W panel
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Global -> register staging: thread t copies chunk (t & 7) of rows (t >> 3) + 32 i.
    const int lr = t >> 3, lc = t & 7;
    const int8_t* ga = A + (int64_t)(m0 + lr) * K + lc * 16;
    const int8_t* gb = B + (int64_t)(n0 + lr) * K + lc * 16;
    const int64_t row_step = (int64_t)32 * K;

    u32x4 ra[LOADS], rb[LOADS];
    auto load_stage = [&](int k0) {
        const bool kin = k0 + lc * 16 < K;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const bool va = kin && (m0 + lr + 32 * i < M);
            const bool vb = kin && (n0 + lr + 32 * i < N);
            ra[i] = va ? *reinterpret_cast<const u32x4*>(ga + i * row_step + k0) : u32x4{0, 0, 0, 0};
            rb[i] = vb ? *reinterpret_cast<const u32x4*>(gb + i * row_step + k0) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_stage = [&](int buf) {
        int8_t* sa = smem + buf * STAGE;
        int8_t* sb = sa + BM * BK;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = lr + 32 * i;
            *reinterpret_cast<u32x4*>(sa + swz(r, lc)) = ra[i];
            *reinterpret_cast<u32x4*>(sb + swz(r, lc)) = rb[i];
        }
    };

    i32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = i32x4{0, 0, 0, 0};

    // Fragment reads: lane l takes row (l & 15) of a 16-row block, 16-byte chunk (l >> 4)
    // of the 64-byte k-substep; the A and B operands use the same k <-> (lane, byte)
    // assignment, so their products pair the same k.
    const int fr = lane & 15, fc = lane >> 4;
    auto compute = [&](int buf) {
        const int8_t* sa = smem + buf * STAGE;
        const int8_t* sb = sa + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 64; ++ks) {
            i32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const i32x4*>(sa + swz(wm * WM + i * 16 + fr, ks * 4 + fc));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const i32x4*>(sb + swz(wn * WN + j * 16 + fr, ks * 4 + fc));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    const int KT = (K + BK - 1) / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more)
            load_stage((kt + 1) * BK);
        compute(kt & 1);
        if (more)
            store_stage((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue. Accumulator element r of tile (i, j) in lane l is C[4 (l >> 4) + r][l & 15]
    // of that 16 x 16 tile.
    const int mb = m0 + wm * WM + 4 * (lane >> 4);
    const int nb = n0 + wn * WN + (lane & 15);
    float wsv[FN], bv[FN];
    if constexpr (YMODE != Y_I32) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = nb + 16 * j;
            wsv[j] = n < N ? ws[n] : 0.0f;
            bv[j] = (bias != nullptr && n < N) ? bias[n] : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb + 16 * i + r;
            if (m >= M)
                continue;
            float xsv = 0.0f;
            if constexpr (YMODE != Y_I32)
                xsv = xs[m];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = nb + 16 * j;
                if (n >= N)
                    continue;
                const int64_t o = (int64_t)m * N + n;
                if constexpr (YMODE == Y_I32) {
                    reinterpret_cast<int32_t*>(Y)[o] = acc[i][j][r];
                } else {
                    const float y = (float)acc[i][j][r] * xsv * wsv[j] + bv[j];
                    if constexpr (YMODE == Y_F32)
                        reinterpret_cast<float*>(Y)[o] = y;
                    else
                        reinterpret_cast<_Float16*>(Y)[o] = (_Float16)y;
                }
            }
        }
    }
}

}  // namespace

ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0)
        return QL_OK;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(NTHR);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (y_mode) {
    case Y_F32:
        hipLaunchKernelGGL(gemm_w8a8_kernel<Y_F32>, grid, block, 0, stream, xq, x_scale, wq, w_scale,
                           bias, y, m, n, k, tiles_m, tiles_n);
        break;
    case Y_F16:
        hipLaunchKernelGGL(gemm_w8a8_kernel<Y_F16>, grid, block, 0, stream, xq, x_scale, wq, w_scale,
                           bias, y, m, n, k, tiles_m, tiles_n);
        break;
    default:
        hipLaunchKernelGGL(gemm_w8a8_kernel<Y_I32>, grid, block, 0, stream, xq, x_scale, wq, w_scale,
                           bias, y, m, n, k, tiles_m, tiles_n);
        break;
    }
    return launch_status();
}

}  // namespace ql
