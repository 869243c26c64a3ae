// wonly.hip -- weight-only quantized GEMM / decode GEMV on gfx950 (W8A16, W4A16).
//
//   y[m,n] = sum_g s[g,n] * sum_{k in g} x[m,k] * (q[k,n] - z[g,n]) + bias[n]
//
// quant67.com ch.17 §四: weight-only quantization keeps weights in HBM as 8- or 4-bit
// codes and dequantizes them on chip, so the decode path moves as few bytes as
// possible; fp32 accumulation (§六). xdnf.cn INT4/FP16 mixed GEMM §3.2 and §4.2: unpack
// the int4 codes by shift and mask, dequantize, multiply with fp16 activations and
// accumulate in fp32. zingnex.cn 核心量化流程: uint8 codes with a zero point and a scale
// per block of 64 weights along K. hotelren.com "量化模型的矩阵乘法": zero is optional
// and present only for the asymmetric format.
//
// Design. Codes are turned into fp16 numbers that are the integers (q - z) exactly:
// an 8-bit offset code u is ORed into the mantissa of fp16 1024.0 (bits 0x6400) giving
// exactly 1024 + u, since the fp16 spacing is 1 on [1024, 2048); subtracting 1024 + z
// (itself exact) leaves u - z with no rounding. Signed codes are first moved to offset
// binary by flipping their sign bit (int8: u = q + 128; int4: u = q + 8). The integer
// weights then enter v_mfma_f32_16x16x32_f16 against fp16 activations, whose products
// are exact in the fp32 accumulator; the scale multiplies each group's partial sum
// rather than each weight.
//
// Work split: a wave owns 16*NT output columns and all M rows (MT blocks of 16); the 4
// waves of a workgroup split the K range (KW ways) and/or the columns (4/KW ways), and
// the K-split partial sums are added through LDS. Weights stream from HBM in batches of
// U steps of 64 k, each batch's loads issued before the previous batch is consumed.
#include "ql_internal.h"

namespace ql {
namespace {

template <int FMT>
struct WBytes {  // weight bytes per lane per step (64 k) per 16-column block
    static constexpr int v = FMT == W_INT4_SYM ? 8 : 16;
};

template <int FMT>
using WReg = typename std::conditional<FMT == W_INT4_SYM, u32x2, u32x4>::type;

// Two 8-bit offset codes (bits 0-7 and 16-23 of v, other bits zero) -> fp16 pair 1024+u.
__device__ inline uint32_t magic_pair(uint32_t v) { return v | 0x64006400u; }

// 16 int8/uint8 codes (k = 16*lg + 0..15 of the step) -> two fp16x8 operands, values
// (code - bias16) where bias16 = 1024 + offset: exact integers.
__device__ inline void bytes_to_f16(const u32x4 w, uint32_t flip, _Float16 sub, f16x8& lo,
                                    f16x8& hi) {
    uint32_t p[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t v = w[d] ^ flip;
        p[2 * d] = magic_pair((v & 0xFFu) | ((v & 0xFF00u) << 8));
        p[2 * d + 1] = magic_pair(((v >> 16) & 0xFFu) | ((v >> 8) & 0xFF0000u));
    }
    const u32x4 a{p[0], p[1], p[2], p[3]}, b{p[4], p[5], p[6], p[7]};
    const f16x8 s{sub, sub, sub, sub, sub, sub, sub, sub};
    lo = __builtin_bit_cast(f16x8, a) - s;
    hi = __builtin_bit_cast(f16x8, b) - s;
}

// One int32 word of eight int4 codes (element j in bits 4j..4j+3) -> fp16x8 in the order
// [q0, q4, q1, q5, q2, q6, q3, q7]; the activation operand uses the same order.
__device__ inline f16x8 int4_to_f16(uint32_t w) {
    const uint32_t v = w ^ 0x88888888u;  // two's complement -> offset binary q + 8
    const u32x4 a{magic_pair(v & 0x000F000Fu), magic_pair((v >> 4) & 0x000F000Fu),
                  magic_pair((v >> 8) & 0x000F000Fu), magic_pair((v >> 12) & 0x000F000Fu)};
    const _Float16 c = (_Float16)1032.0f;
    const f16x8 s{c, c, c, c, c, c, c, c};
    return __builtin_bit_cast(f16x8, a) - s;
}

// Reorders eight consecutive activations x0..x7 to [x0, x4, x1, x5, x2, x6, x3, x7].
__device__ inline f16x8 interleave4(const f16x8 x) {
    return f16x8{x[0], x[4], x[1], x[5], x[2], x[6], x[3], x[7]};
}

template <int FMT, int MT, int NT, int KW, int U>
__global__ __launch_bounds__(256) void wonly_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wc, const void* __restrict__ scale,
    const uint8_t* __restrict__ zp, int group, const float* __restrict__ bias,
    _Float16* __restrict__ Y, int M, int N, int K) {
    constexpr int NW = 4 / KW;
    using WR = WReg<FMT>;
    __shared__ f32x4 red[KW > 1 ? (KW - 1) * NW * MT * NT * 64 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kw = wave % KW, nw = wave / KW;
    const int ln = lane & 15, lg = lane >> 4;
    const int ncol0 = (blockIdx.x * NW + nw) * 16 * NT;
    const int S = K >> 6;
    const int s0 = (kw * S) / KW, s1 = ((kw + 1) * S) / KW;
    const int ngroups = K / group;
    const int64_t wrow = FMT == W_INT4_SYM ? K / 2 : K;   // bytes per weight column

    // Column handled by this lane in block j (clamped for loads; stores are masked).
    const uint8_t* wp[NT];
    int ncl[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = ncol0 + 16 * j + ln;
        ncl[j] = n < N ? n : N - 1;
        wp[j] = Wc + (int64_t)ncl[j] * wrow + lg * WBytes<FMT>::v;
    }
    const _Float16* xp[MT];
    bool xv[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + ln;
        xv[i] = m < M;
        xp[i] = X + (int64_t)(xv[i] ? m : 0) * K + lg * 16;
    }

    f32x4 acc[MT][NT], part[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[i][j] = f32x4{0, 0, 0, 0};
            part[i][j] = f32x4{0, 0, 0, 0};
        }

    auto load = [&](int s, WR (&w)[NT], u32x4 (&x)[MT][2]) {
        const int k0 = s << 6;
#pragma unroll
        for (int j = 0; j < NT; ++j)
            w[j] = *reinterpret_cast<const WR*>(wp[j] + (FMT == W_INT4_SYM ? k0 / 2 : k0));
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (xv[i]) {
                x[i][0] = *reinterpret_cast<const u32x4*>(xp[i] + k0);
                x[i][1] = *reinterpret_cast<const u32x4*>(xp[i] + k0 + 8);
            } else {
                x[i][0] = u32x4{0, 0, 0, 0};
                x[i][1] = u32x4{0, 0, 0, 0};
            }
        }
    };

    auto flush = [&](int g) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float sc;
            if constexpr (FMT == W_INT4_SYM)
                sc = (float)reinterpret_cast<const _Float16*>(scale)[(int64_t)ncl[j] * ngroups + g];
            else
                sc = reinterpret_cast<const float*>(scale)[(int64_t)ncl[j] * ngroups + g];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                acc[i][j] += sc * part[i][j];
                part[i][j] = f32x4{0, 0, 0, 0};
            }
        }
    };

    auto compute = [&](int s, const WR (&w)[NT], const u32x4 (&x)[MT][2]) {
        const int k0 = s << 6;
        const int g = k0 / group;
        f16x8 xa[MT][2];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f16x8 v = __builtin_bit_cast(f16x8, x[i][h]);
                xa[i][h] = FMT == W_INT4_SYM ? interleave4(v) : v;
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f16x8 wb[2];
            if constexpr (FMT == W_INT4_SYM) {
                wb[0] = int4_to_f16(w[j][0]);
                wb[1] = int4_to_f16(w[j][1]);
            } else if constexpr (FMT == W_INT8_SYM) {
                bytes_to_f16(w[j], 0x80808080u, (_Float16)1152.0f, wb[0], wb[1]);
            } else {
                const int z = zp[(int64_t)ncl[j] * ngroups + g];
                bytes_to_f16(w[j], 0u, (_Float16)(float)(1024 + z), wb[0], wb[1]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][h], wb[h], part[i][j], 0, 0, 0);
        }
        if (((k0 + 64) % group) == 0 || s + 1 == s1)
            flush(g);
    };

    WR wa[U][NT], wb2[U][NT];
    u32x4 xa[U][MT][2], xb[U][MT][2];
    auto load_batch = [&](int sb, WR (&w)[U][NT], u32x4 (&x)[U][MT][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (sb + u < s1)
                load(sb + u, w[u], x[u]);
    };
    auto compute_batch = [&](int sb, const WR (&w)[U][NT], const u32x4 (&x)[U][MT][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (sb + u < s1)
                compute(sb + u, w[u], x[u]);
    };

    if (s0 < s1) {
        load_batch(s0, wa, xa);
        for (int sb = s0; sb < s1; sb += 2 * U) {
            if (sb + U < s1)
                load_batch(sb + U, wb2, xb);
            compute_batch(sb, wa, xa);
            if (sb + U < s1) {
                if (sb + 2 * U < s1)
                    load_batch(sb + 2 * U, wa, xa);
                compute_batch(sb + U, wb2, xb);
            }
        }
    }

    // K-split reduction: waves kw > 0 park their sums in LDS, kw == 0 adds them.
    if constexpr (KW > 1) {
        if (kw > 0) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    red[(((kw - 1) * NW + nw) * MT * NT + i * NT + j) * 64 + lane] = acc[i][j];
        }
        __syncthreads();
        if (kw > 0)
            return;
#pragma unroll
        for (int q = 1; q < KW; ++q)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] += red[(((q - 1) * NW + nw) * MT * NT + i * NT + j) * 64 + lane];
    }

    // Output element r of block (i, j) in lane l is C[4 (l >> 4) + r][l & 15].
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = ncol0 + 16 * j + ln;
        if (n >= N)
            continue;
        const float b = bias ? bias[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * i + 4 * lg + r;
                if (m < M)
                    Y[(int64_t)m * N + n] = (_Float16)(acc[i][j][r] + b);
            }
    }
}

template <int FMT, int MT, int NT, int KW, int U>
ql_status launch_cfg(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                     int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                     hipStream_t stream) {
    constexpr int cols = 16 * NT * (4 / KW);
    const dim3 grid((unsigned)((N + cols - 1) / cols)), block(256);
    hipLaunchKernelGGL((wonly_kernel<FMT, MT, NT, KW, U>), grid, block, 0, stream,
                       reinterpret_cast<const _Float16*>(x), reinterpret_cast<const uint8_t*>(codes),
                       scale, zp, (int)group, bias, reinterpret_cast<_Float16*>(y), (int)M, (int)N,
                       (int)K);
    return launch_status();
}

template <int FMT, int MT>
ql_status launch_fmt(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                     int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                     hipStream_t stream) {
    // Batch depth U shrinks as the activation fragments per step grow with MT.
    constexpr int U = MT == 1 ? 4 : (MT == 2 ? 2 : 1);
    // Few columns: split K four ways so that every CU streams part of the weights.
    if (N <= 8192)
        return launch_cfg<FMT, MT, 1, 4, U>(x, codes, scale, zp, group, bias, y, M, N, K, stream);
    return launch_cfg<FMT, MT, 2, 2, U>(x, codes, scale, zp, group, bias, y, M, N, K, stream);
}

template <int FMT>
ql_status launch_rows(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                      int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
    // Rows are processed 64 at a time (MT = 4 blocks of 16); smaller M uses fewer blocks.
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
        const int64_t mc = M - m0 < 64 ? M - m0 : 64;
        const void* xs = reinterpret_cast<const _Float16*>(x) + m0 * K;
        void* ys = reinterpret_cast<_Float16*>(y) + m0 * N;
        ql_status st;
        if (mc <= 16)
            st = launch_fmt<FMT, 1>(xs, codes, scale, zp, group, bias, ys, mc, N, K, stream);
        else if (mc <= 32)
            st = launch_fmt<FMT, 2>(xs, codes, scale, zp, group, bias, ys, mc, N, K, stream);
        else
            st = launch_fmt<FMT, 4>(xs, codes, scale, zp, group, bias, ys, mc, N, K, stream);
        if (st != QL_OK)
            return st;
    }
    return QL_OK;
}

}  // namespace

ql_status launch_wonly(const void* x, const void* codes, int fmt, const void* scale,
                       const uint8_t* zp, int64_t group, const float* bias, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0)
        return QL_OK;
    if (group == 0)
        group = K;
    switch (fmt) {
    case W_INT8_SYM:
        return launch_rows<W_INT8_SYM>(x, codes, scale, zp, group, bias, y, M, N, K, stream);
    case W_UINT8_ZP:
        return launch_rows<W_UINT8_ZP>(x, codes, scale, zp, group, bias, y, M, N, K, stream);
    default:
        return launch_rows<W_INT4_SYM>(x, codes, scale, zp, group, bias, y, M, N, K, stream);
    }
}

}  // namespace ql
