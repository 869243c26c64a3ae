// gemm_w8a8_mid.hip -- the W8A8 layer on 64 x 64 output tiles, for row counts between the
// few-row kernel's and the point where the tile kernel's 128 x 256 and 256 x 256 tiles fill the
// chip; with the tile kernel's epilogues (scales and bias in fp32, fp16 or int32 output,
// zero-point activations, int8 output with static scales, fused activations) and the same
// layer on OCP E4M3 fp8 codes.
//
// The operation is gemm_w8a8.hip's (hotelren.com "量化算法的本质", "W8A8矩阵乘法":
// Y = (x_scale * Xq) @ (w_scale * Wq) + bias, X [M,K] row-major, W [K,N] column-major;
// quant67.com ch.17 §四: exact int32 sums, scales, bias and activation in the epilogue;
// 2048ai.net INT8 Llama-2-7B write-up §5.3: K tiles double-buffered on chip). At M = 256,
// N = 4096 the tile kernel has 32 tiles for 256 CUs; here the same problem has 256.
//
// A workgroup of 4 waves (one per SIMD) owns a 64 x 64 tile; wave w computes the 32 x 32
// block (w & 1, w >> 1) on v_mfma_i32_32x32x32_i8 (fp8: v_mfma_f32_32x32x64_f8f6f4), W's
// fragment as the first operand as in the tile kernel. K advances 128 bytes per stage
// through a ring of four LDS stages filled by direct buffer -> LDS copies (each wave copies
// 16 rows of X and 16 of W per stage); a stage's fragments are read one stage ahead of its
// MFMAs, so LDS reads overlap the matrix cores. One workgroup barrier per stage: after it
// every wave's copies of the next stage have landed, and the buffer the new copies go to
// was last read two stages before. Rows of 128 bytes hold their 16-byte chunks at
// position c ^ h(r), h(r) = (r & 7) ^ ((r >> 3) & 1), so the 32 rows of a fragment read
// fall on distinct bank groups.
#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int MID_T = 64;                     // tile rows and columns
constexpr int MID_BK = 128;                   // bytes of k per stage
constexpr int MID_NS = 4;                     // stages in the ring
constexpr int MID_STAGE = 2 * MID_T * MID_BK;  // X rows then W rows: 16 KiB

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// s_waitcnt immediate: at most n vector-memory operations pending (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// Waits until this wave's copies of a stage have landed, when min(C, n) later stages (CPS
// copies each) were issued after it: the waitcnt immediate for the wave-uniform n.
template <int CPS, int C>
__device__ inline void wait_stages(int n) {
    if constexpr (C <= 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    } else {
        if (n >= C)
            __builtin_amdgcn_s_waitcnt(vmcnt_le(C * CPS));
        else
            wait_stages<CPS, C - 1>(n);
    }
}

__device__ inline int hsw(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at l * 16 past the
// wave-uniform LDS address. An offset past the descriptor's size writes zeros.
__device__ inline void copy16(__amdgpu_buffer_rsrc_t r, int voff, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, 0, 0, 0);
#endif
}

__device__ inline i32x8 cat8m(i32x4 lo, i32x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

template <bool FP8>
using MidAcc = typename std::conditional<FP8, f32x16, i32x16>::type;

struct MidEpi {
    const float* x_zero;     // per row (zero-point activations), or NULL
    const int32_t* colsum;   // W's column code sums (with x_zero)
    const float* out_scale;  // int8 output: 1 or N output scales, or NULL
    int out_scale_n;
};

template <int YMODE, int ACT, bool ASYM, bool FP8>
__global__ __launch_bounds__(256) void gemm_w8a8_mid_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M, int N,
    int K, MidEpi epi, int tiles_m, int ntiles) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[MID_NS * MID_STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tiles dealt to the XCDs in contiguous runs (column-major: neighbours share W)
    const int tile = xcd_remap(blockIdx.x, ntiles);
    const int tn = tile / tiles_m, tm = tile - tn * tiles_m;
    const int m0 = tm * MID_T, n0 = tn * MID_T;
    const int KT = (K + MID_BK - 1) / MID_BK;   // the last stage may be half deep (K % 128 == 64)

    // Copies: wave w moves rows 16 w .. 16 w + 15 of X's and of W's 64 (two copies of 8 rows
    // each); lane l takes row R + (l >> 3) and logical chunk (l & 7) ^ h(row), landing at
    // chunk position l & 7. Rows past M or N read zeros (outside the descriptor).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A) + (int64_t)m0 * K, 0, min(M - m0, MID_T) * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B) + (int64_t)n0 * K, 0, min(N - n0, MID_T) * K, 0x00020000);
    int voff[2];
    const bool half_last = (K & (MID_BK - 1)) != 0;
    int hi[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int r = 16 * wave + 8 * c + (lane >> 3);
        const int chunk = (lane & 7) ^ hsw(r);
        voff[c] = r * K + 16 * chunk;
        // a half-deep last stage reads zeros above its 64 bytes
        hi[c] = half_last && chunk >= 4 ? 0x40000000 : 0;
    }
    auto copies = [&](int kt) {
        int8_t* st = smem + (kt % MID_NS) * MID_STAGE;
        const int cut = kt == KT - 1 ? -1 : 0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int o = (voff[c] + kt * MID_BK) | (hi[c] & cut);
            copy16(ra, o, st + (16 * wave + 8 * c) * MID_BK);
            copy16(rb, o, st + MID_T * MID_BK + (16 * wave + 8 * c) * MID_BK);
        }
    };
    constexpr int CPS = 4;   // copies per stage per wave

    // Fragments: lane l reads row l & 31 of its 32-row block, logical chunk 2 ks + (l >> 5) of
    // substep ks (32 bytes of k).
    const int wm = wave & 1, wn = wave >> 1;
    const int fr = lane & 31;
    i32x4 fa[2][4], fb[2][4];   // [ring of two stages][substep]
    auto read = [&](int kt, int p) {
        const int8_t* st = smem + (kt % MID_NS) * MID_STAGE;
        const int ra_ = 32 * wm + fr, rb_ = 32 * wn + fr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 2 * ks + (lane >> 5);
            fa[p][ks] = *reinterpret_cast<const i32x4*>(st + ra_ * MID_BK + ((c ^ hsw(ra_)) << 4));
            fb[p][ks] = *reinterpret_cast<const i32x4*>(st + (MID_T + rb_) * MID_BK + ((c ^ hsw(rb_)) << 4));
        }
    };
    MidAcc<FP8> acc;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        acc[e] = 0;
    auto mfma = [&](int p) {
        if constexpr (FP8) {
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    cat8m(fb[p][2 * kp], fb[p][2 * kp + 1]), cat8m(fa[p][2 * kp], fa[p][2 * kp + 1]), acc,
                    0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[p][ks], fa[p][ks], acc, 0, 0, 0);
        }
    };

    // Prologue: stages 0 .. NS - 2 in flight; stage 0 landed everywhere, then read.
#pragma unroll
    for (int s = 0; s < MID_NS - 1; ++s)
        if (s < KT)
            copies(s);
    wait_stages<CPS, MID_NS - 2>(KT - 1);   // stages issued after stage 0
    asm volatile("s_barrier" ::: "memory");
    read(0, 0);
    // Stage kt: its fragments are in fa/fb[kt & 1]. Wait for this wave's copies of stage
    // kt + 1, barrier (every wave's copies of kt + 1 landed; every wave is past its reads of
    // stage kt - 1, whose buffer (kt + NS - 1) % NS is refilled next), issue the copies of
    // stage kt + NS - 1, read stage kt + 1, run stage kt's MFMAs. The loop runs two stages
    // per trip so that the fragment parity is a constant.
    auto stage = [&](int kt, auto par) {
        constexpr int P = decltype(par)::value;
        if (kt + 1 < KT)
            wait_stages<CPS, MID_NS - 3>(KT - 2 - kt);   // stages issued after kt + 1
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (kt + MID_NS - 1 < KT)
            copies(kt + MID_NS - 1);
        if (kt + 1 < KT)
            read(kt + 1, 1 - P);
        mfma(P);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < KT; kt += 2) {
        stage(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < KT)
            stage(kt + 1, std::integral_constant<int, 1>{});
    }

    // Epilogue: element e of lane l is C[32 wm + (l & 31)][32 wn + 8 (e >> 2) + 4 (l >> 5) + (e & 3)];
    // rows past M and columns past N are not stored.
    const int m = m0 + 32 * wm + (lane & 31);
    if (m >= M)
        return;
    float xsm = 0.0f, zxm = 0.0f;
    if constexpr (YMODE != Y_I32) {
        xsm = xs[m];
        if constexpr (ASYM)
            zxm = epi.x_zero[m];
    }
    using OutT = typename std::conditional<YMODE == Y_F16, _Float16,
                 typename std::conditional<YMODE == Y_F32, float,
                 typename std::conditional<YMODE == Y_I8, int8_t, int32_t>::type>::type>::type;
    using Out4 = OutT __attribute__((ext_vector_type(4)));
    OutT* yrow = reinterpret_cast<OutT*>(Y) + (int64_t)m * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int c0 = n0 + 32 * wn + 8 * g + 4 * (lane >> 5);
        Out4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * g + q;
            const int n = min(c0 + q, N - 1);
            if constexpr (YMODE == Y_I32) {
                v[q] = acc[e];
            } else {
                const float wsn = ws[n], bn = bias != nullptr ? bias[n] : 0.0f;
                if constexpr (YMODE == Y_I8) {
                    const float so = epi.out_scale[epi.out_scale_n == 1 ? 0 : n];
                    v[q] = requant_code(activation<ACT>(epilogue_unfused((float)acc[e], xsm, wsn, bn)), so, 1.0f / so);
                } else if constexpr (ASYM) {
                    // sum_k (q_x - z_x) q_w = acc - z_x colsum, with one rounding
                    const float t = fmaf(-zxm, (float)epi.colsum[n], (float)acc[e]);
                    v[q] = (OutT)activation<ACT, YMODE == Y_F16>(t * xsm * wsn + bn);
                } else {
                    v[q] = (OutT)activation<ACT, YMODE == Y_F16>((float)acc[e] * xsm * wsn + bn);
                }
            }
        }
        if (c0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<Out4*>(yrow + c0) = v;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c0 + q < N)
                    yrow[c0 + q] = v[q];
        }
    }
}

template <int YMODE, bool ASYM, bool FP8>
void launch_act(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, const float* bias,
                void* y, int act, int M, int N, int K, MidEpi epi, hipStream_t stream) {
    const int tiles_m = (M + MID_T - 1) / MID_T, tiles_n = (N + MID_T - 1) / MID_T;
    const int ntiles = tiles_m * tiles_n;
    const dim3 grid((unsigned)ntiles), block(256);
#define QL_MID(A)                                                                                          \
    hipLaunchKernelGGL((gemm_w8a8_mid_kernel<YMODE, A, ASYM, FP8>), grid, block, 0, stream, xq, xs, wq, ws, \
                       bias, y, M, N, K, epi, tiles_m, ntiles)
    if constexpr (YMODE == Y_I32) {
        QL_MID(ACT_NONE);
    } else {
        if (act == ACT_GELU)
            QL_MID(ACT_GELU);
        else if (act == ACT_SILU)
            QL_MID(ACT_SILU);
        else
            QL_MID(ACT_NONE);
    }
#undef QL_MID
}

}  // namespace

ql_status launch_gemm_w8a8_mid(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const float* bias, void* y, int y_mode, int act,
                               const float* x_zero, const int32_t* colsum, const float* out_scale,
                               int out_scale_n, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                               bool e4m3) {
    if (M == 0 || N == 0)
        return QL_OK;
    const int m = (int)M, n = (int)N, k = (int)K;
    const MidEpi epi{x_zero, colsum, out_scale, out_scale_n};
    if (e4m3) {
        (y_mode == Y_F16 ? launch_act<Y_F16, false, true> : launch_act<Y_F32, false, true>)(
            xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
        return launch_status();
    }
    if (y_mode == Y_I32)
        launch_act<Y_I32, false, false>(xq, x_scale, wq, w_scale, bias, y, ACT_NONE, m, n, k, epi, stream);
    else if (y_mode == Y_I8)
        launch_act<Y_I8, false, false>(xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
    else if (x_zero != nullptr)
        (y_mode == Y_F16 ? launch_act<Y_F16, true, false> : launch_act<Y_F32, true, false>)(
            xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
    else
        (y_mode == Y_F16 ? launch_act<Y_F16, false, false> : launch_act<Y_F32, false, false>)(
            xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
    return launch_status();
}

}  // namespace ql
