// gemm_w8a8_small.hip -- the W8A8 layer for a few rows of X (M <= 128: decode-time batches),
// with the tile kernel's epilogues: scales and bias (fp32, fp16 or int32 output), zero-point
// activations, int8 output with static scales, and the fused activations; and the same layer
// with OCP E4M3 fp8 codes.
//
// The same operation as gemm_w8a8.hip (hotelren.com "量化算法的本质", "W8A8矩阵乘法":
// Y = (x_scale * Xq) @ (w_scale * Wq) + bias; quant67.com ch.17 §四: exact int32 sums, scales,
// bias and activation in the epilogue), laid out for the case where W's bytes dominate: with
// few rows the tile kernel has only N / 256 workgroups, far too few to stream W at HBM rate.
// Here a workgroup owns 16 output columns (N / 16 workgroups), its waves split K, and
// every byte of W is read once, in 64-byte segments per lane quad:
//   - lane l loads 16 bytes of line (l >> 2) (a column of W or a row of X) at byte 16 (l & 3)
//     of a 64-deep k-step, so the four lanes of a quad read one 64-byte segment;
//   - ds_bpermute moves the words to the matrix core's order, where lane l holds line
//     (l & 15) and k-chunk (l >> 4) (the k order inside one step is the same for both operands,
//     which is all the product needs);
//   - v_mfma_i32_16x16x64_i8 accumulates exactly in int32 for up to eight 16-row blocks;
//   - the waves' sums meet in LDS (int32, exact) and the epilogue writes y.
#include <stdint.h>

#include "ql_internal.h"

namespace ql {
namespace {

// SW waves per workgroup. In group mode each wave takes every SW-th group of SU 64-deep
// k-steps and loads a group at once; in ring mode (RING) each wave takes a contiguous range of
// k-steps and keeps SU of them in flight, loading step t + SU as soon as step t is computed.
// With several workgroups per CU (N > 16 x 2 x CUs), four waves of 16-step groups are fastest
// (the resident workgroups overlap one another; a ring measured 7% slower at N = 14336, one
// row). With about one workgroup per CU, eight waves on a ring: with 8-step groups each wave
// issued its whole K range at once (64 KB per CU at K = 4096), and the requests of all CUs came
// back in no useful order. Measured at N = K = 4096 against 8-step groups: one row 6.64 ->
// 5.98 us, 8 rows 7.56 -> 6.62 us (4 steps in flight); 16 rows 7.85 -> 6.93 us, 32 rows 9.04
// -> 8.20 us, 64 rows 13.46 -> 12.02 us (2 steps in flight: from 16 rows X adds as many bytes
// per step as W). The fp8 codes use the same ring over pairs of steps (2 pairs in flight up to
// 8 rows, 1 beyond): 6.85 -> 6.40 us at one row, 9.17 -> 7.94 us at 32 rows, 13.49 -> 11.69 us
// at 64 rows.
constexpr int SCOLS = 16;   // output columns per workgroup

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4s __attribute__((ext_vector_type(4)));

// Operand codes: int8 (exact int32 sums) or OCP E4M3 fp8 (fp32 sums; one 16x16x128 fp8 step
// takes the permuted fragments of two consecutive 64-deep steps, a missing second step being
// zero codes, and E4M3 code 0 is +0).
template <bool FP8>
using SmallAcc = typename std::conditional<FP8, f32x4s, i32x4>::type;

__device__ inline i32x8 cat8s(i32x4 lo, i32x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ inline i32x4 to_mfma_order(i32x4 v, int src_byte) {
    i32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = __builtin_amdgcn_ds_bpermute(src_byte, v[i]);
    return r;
}

// The epilogue's optional terms, as in the tile kernel: the rows' zero points and W's column
// code sums (asymmetric activations), or the output scales of int8 output.
struct SmallEpi {
    const float* x_zero;
    const int32_t* colsum;
    const float* out_scale;
    int out_scale_n;
};

template <int YMODE, int MB, int ACT, bool ASYM, int SW, int SU, bool FP8, bool RING>
__global__ __launch_bounds__(64 * SW) void gemm_w8a8_small_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M, int N,
    int K, SmallEpi epi) {
    using Acc = SmallAcc<FP8>;
    __shared__ Acc red[SW][MB][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * SCOLS;
    // load side: line lane >> 2 at byte (lane & 3) * 16 of each 64-byte step; lines past
    // the end read the last one (their results are never stored)
    const int ln = lane >> 2, kc = (lane & 3) * 16;
    const int8_t* bp = B + (int64_t)min(n0 + ln, N - 1) * K + kc;
    const int8_t* ap[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        ap[b] = A + (int64_t)min(16 * b + ln, M - 1) * K + kc;
    const int src = (((lane & 15) << 2) | (lane >> 4)) * 4;

    Acc acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        acc[b] = Acc{0, 0, 0, 0};
    const int S = K / 64;
    if constexpr (RING && FP8) {
        // fp8: a slot holds a pair of steps (s0 + 2p, s0 + 2p + 1) for one 16x16x128 step, a
        // missing second step being zero codes; SU pairs in flight. The hardware's groups of
        // 8 consecutive k lie within one 64-deep step, so the pairing changes only the order
        // in which fp32 group sums are added.
        const int s0 = wave * S / SW, s1 = (wave + 1) * S / SW, T = s1 - s0, P = (T + 1) / 2;
        i32x4 wv[SU][2], xv[MB][SU][2];
        const i32x4 zero{0, 0, 0, 0};
        auto load = [&](int u, int p) {
            if (p < P) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (2 * p + h < T) {
                        const int64_t off = (int64_t)(s0 + 2 * p + h) * 64;
                        wv[u][h] = *reinterpret_cast<const i32x4*>(bp + off);
#pragma unroll
                        for (int b = 0; b < MB; ++b)
                            xv[b][u][h] = *reinterpret_cast<const i32x4*>(ap[b] + off);
                    }
                }
            }
        };
#pragma unroll
        for (int u = 0; u < SU; ++u)
            load(u, u);
        for (int pb = 0; pb < P; pb += SU) {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int p = pb + u;
                if (p < P) {
                    const bool two = 2 * p + 1 < T;
                    const i32x8 bw = cat8s(to_mfma_order(wv[u][0], src), two ? to_mfma_order(wv[u][1], src) : zero);
#pragma unroll
                    for (int b = 0; b < MB; ++b) {
                        const i32x8 aw = cat8s(to_mfma_order(xv[b][u][0], src), two ? to_mfma_order(xv[b][u][1], src) : zero);
                        acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bw, acc[b], 0, 0, 0, 0, 0, 0);
                    }
                    load(u, p + SU);
                }
            }
        }
    } else if constexpr (RING) {
        const int s0 = wave * S / SW, s1 = (wave + 1) * S / SW, T = s1 - s0;
        i32x4 wv[SU], xv[MB][SU];
        auto load = [&](int u, int t) {
            if (t < T) {
                const int64_t off = (int64_t)(s0 + t) * 64;
                wv[u] = *reinterpret_cast<const i32x4*>(bp + off);
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    xv[b][u] = *reinterpret_cast<const i32x4*>(ap[b] + off);
            }
        };
#pragma unroll
        for (int u = 0; u < SU; ++u)
            load(u, u);
        // t < T is uniform across the wave: every lane takes part in the permutes
        for (int tb = 0; tb < T; tb += SU) {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int t = tb + u;
                if (t < T) {
                    const i32x4 bw = to_mfma_order(wv[u], src);
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(to_mfma_order(xv[b][u], src), bw, acc[b], 0, 0, 0);
                    load(u, t + SU);
                }
            }
        }
    } else
    for (int base = wave * SU; base < S; base += SW * SU) {
        i32x4 wv[SU], xv[MB][SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            if (base + u < S) {
                wv[u] = *reinterpret_cast<const i32x4*>(bp + (int64_t)(base + u) * 64);
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    xv[b][u] = *reinterpret_cast<const i32x4*>(ap[b] + (int64_t)(base + u) * 64);
            }
        }
        // the conditions below are uniform across the wave: every lane takes part in the permutes
        if constexpr (FP8) {
            const i32x4 zero{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < SU; u += 2) {
                if (base + u < S) {
                    const bool two = base + u + 1 < S;
                    const i32x8 bw = cat8s(to_mfma_order(wv[u], src), two ? to_mfma_order(wv[u + 1], src) : zero);
#pragma unroll
                    for (int b = 0; b < MB; ++b) {
                        const i32x8 aw = cat8s(to_mfma_order(xv[b][u], src),
                                               two ? to_mfma_order(xv[b][u + 1], src) : zero);
                        acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bw, acc[b], 0, 0, 0, 0, 0, 0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                if (base + u < S) {
                    const i32x4 bw = to_mfma_order(wv[u], src);
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(to_mfma_order(xv[b][u], src), bw, acc[b], 0, 0, 0);
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < MB; ++b)
        red[wave][b][lane] = acc[b];
    __syncthreads();
    const int n = n0 + (lane & 15);
    if (n >= N)
        return;
    float wsn = 0.0f, bn = 0.0f, csn = 0.0f, son = 0.0f, orn = 0.0f;
    if constexpr (YMODE != Y_I32) {
        wsn = ws[n];
        bn = bias != nullptr ? bias[n] : 0.0f;
    }
    if constexpr (ASYM)
        csn = (float)epi.colsum[n];   // exact: |sum| <= 128 K < 2^24
    if constexpr (YMODE == Y_I8) {
        son = epi.out_scale[epi.out_scale_n == 1 ? 0 : n];
        orn = 1.0f / son;
    }
    // wave w finishes row blocks w, w + SW, ...: element i of lane l is C[4 (l >> 4) + i][l & 15]
    auto put_float = [&](int64_t o, float v) {
        if constexpr (YMODE == Y_F16)
            reinterpret_cast<_Float16*>(Y)[o] = (_Float16)v;
        else
            reinterpret_cast<float*>(Y)[o] = v;
    };
    for (int b = wave; b < MB; b += SW) {
        Acc t = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < SW; ++w)
            t += red[w][b][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * b + 4 * (lane >> 4) + i;
            if (m >= M)
                continue;
            const int64_t o = (int64_t)m * N + n;
            if constexpr (YMODE == Y_I32) {
                reinterpret_cast<int32_t*>(Y)[o] = t[i];
            } else if constexpr (YMODE == Y_I8) {
                reinterpret_cast<int8_t*>(Y)[o] =
                    requant_code(activation<ACT>(epilogue_unfused((float)t[i], xs[m], wsn, bn)), son, orn);
            } else if constexpr (ASYM) {
                // sum_k (q_x - z_x) q_w = acc - z_x colsum, with one rounding
                const float ta = fmaf(-epi.x_zero[m], csn, (float)t[i]);
                put_float(o, activation<ACT, YMODE == Y_F16>(ta * xs[m] * wsn + bn));
            } else {
                put_float(o, activation<ACT, YMODE == Y_F16>((float)t[i] * xs[m] * wsn + bn));
            }
        }
    }
}

template <int YMODE, int ACT, bool ASYM, int SW, int SU, bool FP8, bool RING = false>
void launch_mb(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, const float* bias,
               void* y, int M, int N, int K, SmallEpi epi, hipStream_t stream) {
    const dim3 grid((unsigned)((N + SCOLS - 1) / SCOLS)), block(64 * SW);
    const int mb = (M + 15) / 16;
#define QL_SMALL(MBV)                                                                                         \
    hipLaunchKernelGGL((gemm_w8a8_small_kernel<YMODE, MBV, ACT, ASYM, SW, SU, FP8, RING>), grid, block, 0, stream, \
                       xq, xs, wq, ws, bias, y, M, N, K, epi)
    if (mb == 1)
        QL_SMALL(1);
    else if (mb == 2)
        QL_SMALL(2);
    else if (mb == 3)
        QL_SMALL(3);
    else
        QL_SMALL(4);
#undef QL_SMALL
}

// 65 to 128 rows: eight row blocks on eight waves of 4-step groups (X's registers stay within
// limits; the LDS reduction takes 64 KB). Eight waves measured 10-14% faster than four.
template <int YMODE, int ACT, bool ASYM, bool FP8>
void launch_mb8(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, const float* bias,
                void* y, int M, int N, int K, SmallEpi epi, hipStream_t stream) {
    const dim3 grid((unsigned)((N + SCOLS - 1) / SCOLS)), block(64 * 8);
    const int mb = (M + 15) / 16;
#define QL_SMALL8(MBV)                                                                                    \
    hipLaunchKernelGGL((gemm_w8a8_small_kernel<YMODE, MBV, ACT, ASYM, 8, 4, FP8, false>), grid, block, 0, stream, \
                       xq, xs, wq, ws, bias, y, M, N, K, epi)
    if (mb <= 6)
        QL_SMALL8(6);
    else
        QL_SMALL8(8);
#undef QL_SMALL8
}

template <int YMODE, int ACT, bool ASYM, bool FP8>
void launch_shape(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, const float* bias,
                  void* y, int M, int N, int K, SmallEpi epi, hipStream_t stream) {
    const int64_t wgs = (N + SCOLS - 1) / SCOLS;
    if (M > 64)
        launch_mb8<YMODE, ACT, ASYM, FP8>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else if (wgs > 2 * (int64_t)cu_count())
        launch_mb<YMODE, ACT, ASYM, 4, 16, FP8>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else if (FP8 && M <= 8)
        launch_mb<YMODE, ACT, ASYM, 8, 2, true, true>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else if (FP8)
        launch_mb<YMODE, ACT, ASYM, 8, 1, true, true>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else if (M <= 8)
        launch_mb<YMODE, ACT, ASYM, 8, 4, false, true>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else
        launch_mb<YMODE, ACT, ASYM, 8, 2, false, true>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
}

template <int YMODE, bool ASYM, bool FP8 = false>
void launch_act(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, const float* bias,
                void* y, int act, int M, int N, int K, SmallEpi epi, hipStream_t stream) {
    if (act == ACT_GELU)
        launch_shape<YMODE, ACT_GELU, ASYM, FP8>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else if (act == ACT_SILU)
        launch_shape<YMODE, ACT_SILU, ASYM, FP8>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
    else
        launch_shape<YMODE, ACT_NONE, ASYM, FP8>(xq, xs, wq, ws, bias, y, M, N, K, epi, stream);
}

}  // namespace

ql_status launch_gemm_w8a8_small(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                 const float* w_scale, const float* bias, void* y, int y_mode, int act,
                                 const float* x_zero, const int32_t* colsum, const float* out_scale,
                                 int out_scale_n, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                                 bool e4m3) {
    if (M == 0 || N == 0)
        return QL_OK;
    const int m = (int)M, n = (int)N, k = (int)K;
    const SmallEpi epi{x_zero, colsum, out_scale, out_scale_n};
    if (e4m3) {
        (y_mode == Y_F16 ? launch_act<Y_F16, false, true> : launch_act<Y_F32, false, true>)(
            xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
        return launch_status();
    }
    if (y_mode == Y_I32)
        launch_shape<Y_I32, ACT_NONE, false, false>(xq, x_scale, wq, w_scale, bias, y, m, n, k, epi, stream);
    else if (y_mode == Y_I8)
        launch_act<Y_I8, false>(xq, x_scale, wq, w_scale, bias, y, act, m, n, k, epi, stream);
    else if (x_zero != nullptr)
        (y_mode == Y_F16 ? launch_act<Y_F16, true> : launch_act<Y_F32, true>)(xq, x_scale, wq, w_scale, bias, y,
                                                                             act, m, n, k, epi, stream);
    else
        (y_mode == Y_F16 ? launch_act<Y_F16, false> : launch_act<Y_F32, false>)(xq, x_scale, wq, w_scale, bias,
                                                                               y, act, m, n, k, epi, stream);
    return launch_status();
}

}  // namespace ql
