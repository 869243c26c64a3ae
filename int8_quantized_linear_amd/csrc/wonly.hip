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
// Design. Decode is bound by HBM bandwidth, and at these sizes by how many bytes are in
// flight: a CU's share of the weights (64 KB for 4096 x 4096 int8 over 256 CUs) is about
// what HBM latency times the CU's share of bandwidth asks for. So each wave keeps a ring
// of D k-steps of loads in flight in registers, issued D steps ahead of use, and the
// columns are spread so that every CU gets a share (a workgroup covers ceil(N / CUs)
// columns, rounded up to 8; its 4 waves split K four ways).
//
// Codes are turned into fp16 numbers that are the integers (q - z) exactly: an 8-bit
// offset code u is placed in the low byte of fp16 1024.0 (bits 0x6400), giving exactly
// 1024 + u since the fp16 spacing is 1 on [1024, 2048); subtracting 1024 + z (itself
// exact) leaves u - z with no rounding. Signed codes are first moved to offset binary by
// flipping their sign bit (int8: u = q + 128; int4: u = q + 8). The integer weights then
// enter v_mfma_f32_16x16x32_f16 against fp16 activations, whose products are exact in
// the fp32 accumulator; the scale multiplies each group's partial sum rather than each
// weight.
//
// Loads go through buffer descriptors: a lane whose column is past N, a row past M, or
// a step past the wave's K range gets an offset beyond the descriptor's size, and the
// hardware returns zeros without touching memory, so the ring needs no branches.
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int OOB = 0x7FFFFFF0;   // an offset past every descriptor size used here

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             (int)(bytes < OOB ? bytes : OOB), 0x00020000);
}

// Four offset-binary bytes of v -> two fp16 pairs {1024 + b0, 1024 + b1} and
// {1024 + b2, 1024 + b3}: v_perm_b32 interleaves v's bytes with the exponent byte 0x64.
__device__ inline uint32_t magic_lo(uint32_t v) { return __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u); }
__device__ inline uint32_t magic_hi(uint32_t v) { return __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u); }

// 16 codes (k = 16 lg + 0..15 of the step) -> two fp16x8 operands with values
// (code ^ flip) - (sub - 1024): exact integers.
__device__ inline void bytes_to_f16(const u32x4 w, uint32_t flip, _Float16 sub, f16x8& lo,
                                    f16x8& hi) {
    uint32_t p[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t v = w[d] ^ flip;
        p[2 * d] = magic_lo(v);
        p[2 * d + 1] = magic_hi(v);
    }
    const u32x4 a{p[0], p[1], p[2], p[3]}, b{p[4], p[5], p[6], p[7]};
    const f16x8 s{sub, sub, sub, sub, sub, sub, sub, sub};
    lo = __builtin_bit_cast(f16x8, a) - s;
    hi = __builtin_bit_cast(f16x8, b) - s;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// One int32 word of eight int4 codes (element j in bits 4j..4j+3, two's complement) ->
// fp16x8 [q0, q4, q1, q5, q2, q6, q3, q7], exactly. For a nibble n the offset code is
// u = q + 8 = n ^ 8. Masking a nibble pair and XORing with the fp16 pattern of 1024 (with
// bit 3 of each nibble field set) gives in one bitwise step the fp16 pair 1024 + u (low
// nibbles of a byte) or 1024 + 16 u (high nibbles; the fp16 spacing on [1024, 2048) is 1, so
// both are exact); then q = (1024 + u) - 1032 and q = (1024 + 16 u) / 16 - 72, each one
// exact packed fp16 operation.
__device__ inline f16x8 int4_to_f16(uint32_t w) {
    const uint32_t w8 = w >> 8;
    const f16x2 lo_sub{(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 hi_mul{(_Float16)0.0625f, (_Float16)0.0625f}, hi_add{(_Float16)-72.0f, (_Float16)-72.0f};
    const f16x2 a = __builtin_bit_cast(f16x2, (w & 0x000F000Fu) ^ 0x64086408u) - lo_sub;     // q0, q4
    const f16x2 b = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w & 0x00F000F0u) ^ 0x64806480u),
                                              hi_mul, hi_add);                            // q1, q5
    const f16x2 c = __builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) ^ 0x64086408u) - lo_sub;    // q2, q6
    const f16x2 d = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) ^ 0x64806480u),
                                              hi_mul, hi_add);                            // q3, q7
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Reorders eight consecutive activations x0..x7 to [x0, x4, x1, x5, x2, x6, x3, x7].
__device__ inline f16x8 interleave4(const f16x8 x) {
    return f16x8{x[0], x[4], x[1], x[5], x[2], x[6], x[3], x[7]};
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// 4 bytes per lane from global memory straight into LDS (global_load_lds_dword): lane l's
// word lands at l * 4 past the wave-uniform LDS address. Device pass only (in the host
// pass the builtin makes clang drop the kernel's launch stub).
__device__ inline void lds_copy4(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 4, 0, 0);
#endif
}

// s_waitcnt immediate: at most n vector-memory operations pending (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// Step geometry. A step covers KS k of a column; a lane holds KSL = KS / 4 consecutive k
// of it (HN = KS / 32 octets of 8 codes, WB bytes), and the step's MFMA chain per block is
// HN deep: octet h of lane (ln, lg) is k = KSL lg + 8 h + (0..7), paired with the same k
// of the activations.
template <int FMT, int KS>
struct Geo {
    static constexpr int HN = KS / 32;
    static constexpr int KSL = KS / 4;
    static constexpr int WB = FMT == W_INT4_SYM ? KSL / 2 : KSL;
    static constexpr int WSTEP = FMT == W_INT4_SYM ? KS / 2 : KS;   // bytes of a column per step
    using WR = typename std::conditional<WB == 16, u32x4, u32x2>::type;
    static_assert(WB == 8 || WB == 16, "a lane loads 8 or 16 bytes of a column per step");
};

// Scales (and zero points) of the workgroup's columns, staged in LDS when they fit.
constexpr int SL_WORDS = 8192;   // 32 KB

// Ring depth: as many k-steps of loads in flight as fit in about 250 registers per lane
// beside the accumulators and the operands of the step being computed, as a power of two
// (at most 16) so that it divides a wave's step count when K is a multiple of 4 * KS * D
// (the loop is padded to whole rings with zero-filled steps).
template <int FMT, int KS, int MT, int NT, bool GLOAD, int NW>
constexpr int ring_depth() {
    using G = Geo<FMT, KS>;
    constexpr int per_step = NT * (G::WB / 4) + MT * G::HN * 4 + (GLOAD ? NT * (FMT == W_UINT8_ZP ? 2 : 1) : 0);
    constexpr int fixed = MT * NT * 4 + MT * G::HN * 4 + 12 + NT * 2 + MT + 24;
    // one wave per SIMD (NW = 4) may use about 280 registers (VGPRs and AGPRs); two
    // (NW = 8) share the file and get about 200 each
    constexpr int d = ((NW == 4 ? 280 : 200) - fixed) / per_step;
    return d >= 16 ? 16 : d >= 8 ? 8 : d >= 4 ? 4 : 2;
}

// One workgroup of NW waves: `cols` (<= 16 NT) consecutive columns from col0, all M
// (<= 16 MT) rows. Wave w runs k-steps [s0, s1) (its 1/NW of K); lane (ln, lg) = (l & 15, l >> 4) handles
// column col0 + 16 j + ln of block j. SCALES: 0 = one scale per column (applied at the
// end), 1 = per group, staged in LDS, 2 = per group, loaded from global memory each step
// (blocks too large for LDS).
template <int FMT, int KS, int MT, int NT, int SCALES, int D, int NW>
__global__ __launch_bounds__(64 * NW) void wonly_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wc, const void* __restrict__ scale,
    const uint8_t* __restrict__ zp, int group, const float* __restrict__ bias,
    _Float16* __restrict__ Y, int M, int N, int K, int cols) {
    using G = Geo<FMT, KS>;
    using WR = typename G::WR;
    constexpr int HN = G::HN;
    constexpr bool GROUPED = SCALES != 0;
    constexpr bool ZP = FMT == W_UINT8_ZP;
    constexpr int SB = FMT == W_INT4_SYM ? 2 : 4;   // bytes per scale
    __shared__ f32x4 red[NW * MT * NT * 64];
    __shared__ uint32_t sl[SCALES == 1 ? SL_WORDS : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int col0 = blockIdx.x * cols;
    const int ncols = min(cols, N - col0);
    const int S = K / KS;
    const int s0 = wave * S / NW, s1 = (wave + 1) * S / NW;
    const int T = s1 - s0;                       // this wave's steps
    const int TP = (T + D - 1) / D * D;          // padded to whole rings (extra steps load zeros)
    const int ngroups = K / group;
    const int spg = group / KS;                  // steps per group
    const int wrow = FMT == W_INT4_SYM ? K / 2 : K;   // bytes per weight column

    // The block of scales (and zero points) of this workgroup's columns is contiguous:
    // [ncols][ngroups]. With SCALES == 1 it is copied into LDS by direct copies issued
    // before anything else, so the wait for them below does not wait for the weights.
    const int sbytes = ncols * ngroups * SB, zbytes = ZP ? ncols * ngroups : 0;
    const int swords = (sbytes + 3) >> 2, zwords = (zbytes + 3) >> 2;
    if constexpr (SCALES == 1) {
        // Words past the block's last are copies of its last word (never read); the last
        // word may hold up to 3 bytes past the array's end, inside the same aligned word.
        const uint8_t* sg = reinterpret_cast<const uint8_t*>(scale) + (int64_t)col0 * ngroups * SB;
        for (int q0 = wave * 64; q0 < swords; q0 += 64 * NW)
            lds_copy4(sg + 4 * min(q0 + lane, swords - 1), sl + q0);
        if constexpr (ZP) {
            const uint8_t* zg = zp + (int64_t)col0 * ngroups;
            const int zw0 = (swords + 63) & ~63;
            for (int q0 = wave * 64; q0 < zwords; q0 += 64 * NW)
                lds_copy4(zg + 4 * min(q0 + lane, zwords - 1), sl + zw0 + q0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    const __amdgpu_buffer_rsrc_t wr = rsrc(Wc + (int64_t)col0 * wrow, (int64_t)ncols * wrow);
    const __amdgpu_buffer_rsrc_t xr = rsrc(X, (int64_t)M * K * 2);
    const __amdgpu_buffer_rsrc_t sr =
        rsrc(reinterpret_cast<const uint8_t*>(scale) + (int64_t)col0 * ngroups * SB, sbytes);
    const __amdgpu_buffer_rsrc_t zr = rsrc(zp + (int64_t)col0 * ngroups, zbytes);
    // Per-lane byte offsets (below 2^30); the step's part is wave-uniform and goes in the
    // scalar offset. A lane outside the columns or rows gets OOB, which stays past every
    // descriptor size when the step's bytes (below 2^22) are added, so the hardware
    // returns zeros.
    int woff[NT], soff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int c = 16 * j + ln;
        woff[j] = c < ncols ? c * wrow + s0 * G::WSTEP + lg * G::WB : OOB;
        soff[j] = min(c, ncols - 1) * ngroups;   // clamped column: scale and zero index
    }
    int xoff[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + ln;
        xoff[i] = m < M ? m * K * 2 + s0 * KS * 2 + lg * G::KSL * 2 : OOB;
    }

    WR w[D][NT];
    u32x4 x[D][MT][HN];
    float sc[D][NT];
    int zq[D][NT];
    // group of the next step loaded, and the step within it (loads come in step order)
    int gcur = s0 / spg, grem = s0 - gcur * spg;
    auto next_group = [&]() {
        // clamped for the zero-filled steps past the range
        const int g = __builtin_amdgcn_readfirstlane(min(gcur, ngroups - 1));
        const bool wrap = grem + 1 == spg;
        grem = wrap ? 0 : grem + 1;
        gcur += wrap ? 1 : 0;
        return g;
    };
    // Ring slot u <- step t of this wave (zeros past T).
    auto load = [&](int u, int t) {
        // past the range: OR every offset up to OOB or beyond (a uniform mask, so that the
        // compiler keeps one straight-line path)
        const int oob = __builtin_amdgcn_readfirstlane(t < T ? 0 : OOB);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int vo = woff[j] | oob;
            if constexpr (G::WB == 8)
                w[u][j] = __builtin_bit_cast(WR, __builtin_amdgcn_raw_buffer_load_b64(wr, vo, t * G::WSTEP, 0));
            else
                w[u][j] = __builtin_bit_cast(WR, __builtin_amdgcn_raw_buffer_load_b128(wr, vo, t * G::WSTEP, 0));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int vo = xoff[i] | oob;
#pragma unroll
            for (int h = 0; h < HN; ++h)
                x[u][i][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo + h * 16, t * KS * 2, 0));
        }
        if constexpr (SCALES == 2) {
            const int g = next_group();
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if constexpr (FMT == W_INT4_SYM)
                    sc[u][j] = (float)__builtin_bit_cast(
                        _Float16, __builtin_amdgcn_raw_buffer_load_b16(sr, soff[j] * SB, g * SB, 0));
                else
                    sc[u][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, soff[j] * SB, g * SB, 0));
                if constexpr (ZP)
                    zq[u][j] = __builtin_amdgcn_raw_buffer_load_b8(zr, soff[j], g, 0);
            }
        }
    };
    // With SCALES == 1 the step's scale and zero come from LDS when it is computed.
    auto lds_scales = [&](int u) {
        const int g = next_group();
        const int zw0 = (swords + 63) & ~63;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int e = soff[j] + g;
            if constexpr (FMT == W_INT4_SYM)
                sc[u][j] = (float)reinterpret_cast<const _Float16*>(sl)[e];
            else
                sc[u][j] = reinterpret_cast<const float*>(sl)[e];
            if constexpr (ZP)
                zq[u][j] = reinterpret_cast<const uint8_t*>(sl + zw0)[e];
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = f32x4{0, 0, 0, 0};

    auto compute = [&](int u) {
        // the next step's scales are read from LDS one step ahead, so that their latency
        // hides behind this step's work
        if constexpr (SCALES == 1)
            lds_scales((u + 1) % D);
        f16x8 xa[MT][HN];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int h = 0; h < HN; ++h) {
                const f16x8 v = __builtin_bit_cast(f16x8, x[u][i][h]);
                xa[i][h] = FMT == W_INT4_SYM ? interleave4(v) : v;
            }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f16x8 wb[HN];
            if constexpr (FMT == W_INT4_SYM) {
#pragma unroll
                for (int h = 0; h < HN; ++h)
                    wb[h] = int4_to_f16(w[u][j][h]);
            } else if constexpr (FMT == W_INT8_SYM) {
                bytes_to_f16(w[u][j], 0x80808080u, (_Float16)1152.0f, wb[0], wb[1]);
            } else {
                bytes_to_f16(w[u][j], 0u, (_Float16)(float)(1024 + zq[u][j]), wb[0], wb[1]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if constexpr (GROUPED) {
                    f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][0], wb[0], f32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int h = 1; h < HN; ++h)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][h], wb[h], p, 0, 0, 0);
                    acc[i][j] += sc[u][j] * p;
                } else {
#pragma unroll
                    for (int h = 0; h < HN; ++h)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][h], wb[h], acc[i][j], 0, 0, 0);
                }
            }
        }
    };

#pragma unroll
    for (int u = 0; u < D; ++u)
        load(u, u);
    if constexpr (SCALES == 1) {
        // This wave's copies into LDS are older than the D steps of loads just issued; then
        // the barrier makes every wave's copies visible.
        constexpr int younger = D * (NT + MT * HN);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(younger < 63 ? younger : 63));
        asm volatile("s_barrier" ::: "memory");
        lds_scales(0);
    }
    // sched_barrier keeps each step's work together, so that the registers of one step's
    // products are free before the next step starts.
    for (int tb = 0; tb + D < TP; tb += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            compute(u);
            load(u, tb + D + u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
        compute(u);
        __builtin_amdgcn_sched_barrier(0);
    }

    // The waves' partial sums meet in LDS; wave w then finishes blocks b = w (mod NW).
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            red[((wave * MT + i) * NT + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    // Output element r of block (i, j) in lane l is C[4 (l >> 4) + r][l & 15].
#pragma unroll
    for (int b = 0; b < MT * NT; ++b) {
        if (b % NW != wave)
            continue;
        const int i = b / NT, j = b % NT;
        f32x4 v = red[b * 64 + lane];
#pragma unroll
        for (int q = 1; q < NW; ++q)
            v += red[(q * MT * NT + b) * 64 + lane];
        const int c = 16 * j + ln;
        if (c >= ncols)
            continue;
        const int n = col0 + c;
        if constexpr (!GROUPED)
            v *= reinterpret_cast<const float*>(scale)[n];
        const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m < M)
                Y[(int64_t)m * N + n] = (_Float16)(v[r] + bb);
        }
    }
}

int cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

template <int FMT, int KS, int MT, int NT, int SCALES, int NW>
ql_status launch_cfg(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                     int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                     int cols, hipStream_t stream) {
    constexpr int D = ring_depth<FMT, KS, MT, NT, SCALES == 2, NW>();
    const dim3 grid((unsigned)((N + cols - 1) / cols)), block(64 * NW);
    hipLaunchKernelGGL((wonly_kernel<FMT, KS, MT, NT, SCALES, D, NW>), grid, block, 0, stream,
                       reinterpret_cast<const _Float16*>(x), reinterpret_cast<const uint8_t*>(codes),
                       scale, zp, (int)group, bias, reinterpret_cast<_Float16*>(y), (int)M, (int)N,
                       (int)K, cols);
    return launch_status();
}

template <int FMT, int KS, int MT, int SCALES>
ql_status launch_nt(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                    int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                    int cols, hipStream_t stream) {
    // Two waves per SIMD where one wave's registers cannot hold enough steps in flight.
    constexpr int NW = MT == 2 ? 8 : 4;
    if (cols <= 16)
        return launch_cfg<FMT, KS, MT, 1, SCALES, NW>(x, codes, scale, zp, group, bias, y, M, N, K, cols, stream);
    if (cols <= 32)
        return launch_cfg<FMT, KS, MT, 2, SCALES, NW>(x, codes, scale, zp, group, bias, y, M, N, K, cols, stream);
    return launch_cfg<FMT, KS, MT, 4, SCALES, NW>(x, codes, scale, zp, group, bias, y, M, N, K, cols, stream);
}

template <int FMT, int KS, int MT>
ql_status launch_mt(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                    int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                    bool grouped, hipStream_t stream) {
    // Columns per workgroup: an equal share per CU, in multiples of 8, at most 64.
    int64_t cols = (N + cu_count() - 1) / cu_count();
    cols = (cols + 7) / 8 * 8;
    if (cols > 64)
        cols = 64;
    if (!grouped)
        return launch_nt<FMT, KS, MT, 0>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, stream);
    // The scale block (and zero-point block after it, at a 64-word boundary) must fit in LDS.
    const int64_t ng = K / group, sb = FMT == W_INT4_SYM ? 2 : 4;
    const int64_t words = ((cols * ng * sb + 3) / 4 + 63) / 64 * 64 + (FMT == W_UINT8_ZP ? (cols * ng + 3) / 4 : 0);
    if (words + 63 <= SL_WORDS)
        return launch_nt<FMT, KS, MT, 1>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, stream);
    return launch_nt<FMT, KS, MT, 2>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, stream);
}

template <int FMT, int KS>
ql_status launch_rows(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                      int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                      bool grouped, hipStream_t stream) {
    // Rows are processed 64 at a time (MT = 4 blocks of 16); smaller M uses fewer blocks.
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
        const int64_t mc = M - m0 < 64 ? M - m0 : 64;
        const void* xs = reinterpret_cast<const _Float16*>(x) + m0 * K;
        void* ys = reinterpret_cast<_Float16*>(y) + m0 * N;
        ql_status st;
        if (mc <= 16)
            st = launch_mt<FMT, KS, 1>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, stream);
        else if (mc <= 32)
            st = launch_mt<FMT, KS, 2>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, stream);
        else
            st = launch_mt<FMT, KS, 4>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, stream);
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
    switch (fmt) {
    case W_INT8_SYM:
        if (group == 0 || group == K)
            return launch_rows<W_INT8_SYM, 64>(x, codes, scale, zp, K, bias, y, M, N, K, false, stream);
        return launch_rows<W_INT8_SYM, 64>(x, codes, scale, zp, group, bias, y, M, N, K, true, stream);
    case W_UINT8_ZP:
        return launch_rows<W_UINT8_ZP, 64>(x, codes, scale, zp, group == 0 ? K : group, bias, y, M, N,
                                           K, true, stream);
    default:
        // 128-k steps (16-byte loads) when a step never straddles a group
        if (group % 128 == 0 && K % 128 == 0)
            return launch_rows<W_INT4_SYM, 128>(x, codes, scale, zp, group, bias, y, M, N, K, true, stream);
        return launch_rows<W_INT4_SYM, 64>(x, codes, scale, zp, group, bias, y, M, N, K, true, stream);
    }
}

}  // namespace ql
