// quant.hip -- quantizer kernels for gfx950.
//
// Per-row symmetric int8 (activations per token, weights per output channel), and the
// producers of the block-asymmetric uint8 and per-group int4 weight formats.
//
// All are HBM-bound streaming kernels: each element is read once from HBM and its code
// written once. Codes are decided in fp32 from the correctly rounded quotient (this file
// is compiled without fast-math, so `a / b` is the IEEE quotient; the per-row kernel
// reaches the same quotient through the row's reciprocal, see code_u8_biased) and
// v_rndne (rintf, round half to even), the precision and rounding of the definitions:
//   scale = max|x| / 127, q = round(x / scale), codes in [-127, 127]
//       2048ai.net INT8 Llama-2-7B write-up §2.2; quant67.com ch.17 §二
//   absmax along the row, clamp_min(1e-10), torch.round (half to even)
//       hotelren.com "量化算法的本质", per_channel_quant_int8
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int QT = 256;       // threads per row-quantizer workgroup
// 16-byte chunks per thread kept in registers: QC_SHORT for rows of up to QT * QC_SHORT
// chunks (8192 fp16 values), QC_LONG for longer rows (up to 16384 fp16 values stay in
// registers, as for Llama-7B's 11008- and 14336-wide activations); the launchers pick one.
// More chunks than a row needs cost the short rows some speed, so both are kept.
constexpr int QC_SHORT = 4;
constexpr int QC_LONG = 8;

__device__ inline float block_max(float v, float* red) {
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, WAVE));
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < QT / WAVE; ++i)
        r = fmaxf(r, red[i]);
    return r;
}

// rint(x / s) clamped to [-127, 127], as (code + 128) in the byte `sel` of `acc`.
// x / s is taken as q0 = RN(x * y), r = x - q0 * s (exact, one fma), RN(q0 + r * y) with
// y = RN(1 / s) divided once per row: Markstein's theorem on division through a correctly
// rounded reciprocal makes that the correctly rounded quotient (a zero may change sign,
// which no code sees), so the code is the one the IEEE quotient gives, at three
// operations instead of a full division.
__device__ inline uint32_t code_u8_biased(float x, float s, float y, uint32_t sel, uint32_t acc) {
    const float q0 = __fmul_rn(x, y);
    const float r = fmaf(-q0, s, x);
    const float q = rintf(fmaf(r, y, q0));
    const float c = __builtin_amdgcn_fmed3f(q, -127.0f, 127.0f) + 128.0f;
    return __builtin_amdgcn_cvt_pk_u8_f32(c, sel, acc);
}

// Asymmetric: rint(x / s + z) clamped to [-128, 127], as (code + 128) in the byte `sel` of
// `acc`. The quotient is the correctly rounded one (as in code_u8_biased), then z is added
// with its own rounding, the two fp32 operations of x / s + z.
__device__ inline uint32_t code_u8_asym(float x, float s, float y, float z, uint32_t sel, uint32_t acc) {
    const float q0 = __fmul_rn(x, y);
    const float r = fmaf(-q0, s, x);
    const float d = fmaf(r, y, q0);   // x / s, correctly rounded
    const float q = rintf(__fadd_rn(d, z));
    const float c = __builtin_amdgcn_fmed3f(q, -128.0f, 127.0f) + 128.0f;
    return __builtin_amdgcn_cvt_pk_u8_f32(c, sel, acc);
}

// Block-wide maximum of hi and of -lo together (one pair of LDS slots per wave).
__device__ inline void block_minmax(float& lo, float& hi, float* red) {
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) {
        hi = fmaxf(hi, __shfl_xor(hi, o, WAVE));
        lo = fminf(lo, __shfl_xor(lo, o, WAVE));
    }
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) {
        red[2 * w] = hi;
        red[2 * w + 1] = lo;
    }
    __syncthreads();
    hi = red[0];
    lo = red[1];
#pragma unroll
    for (int i = 1; i < QT / WAVE; ++i) {
        hi = fmaxf(hi, red[2 * i]);
        lo = fminf(lo, red[2 * i + 1]);
    }
}

// One 16-byte chunk of input as fp32 values: 8 fp16 or 4 fp32 elements.
template <bool F16>
struct Chunk {
    static constexpr int E = F16 ? 8 : 4;
    float v[E];
    __device__ inline void load(const void* p) {
        if constexpr (F16) {
            const f16x8 h = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = (float)h[i];
        } else {
            const f32x4 f = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = f[i];
        }
    }
    __device__ inline float absmax() const {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i)
            a = fmaxf(a, fabsf(v[i]));
        return a;
    }
    __device__ inline void minmax(float& lo, float& hi) const {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            lo = fminf(lo, v[i]);
            hi = fmaxf(hi, v[i]);
        }
    }
    // fp8 (OCP E4M3) codes: the correctly rounded quotient (as code_u8_biased), kept within
    // +-448 (it cannot pass it: s = absmax / 448), then v_cvt_pk_fp8_f32, which rounds to
    // nearest even into E4M3 (gfx950 converts to the OCP format).
    __device__ inline void store_codes_e4m3(uint8_t* q, float s, float y) const {
        uint32_t w[E / 4];
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
            float t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = v[4 * j + i];
                const float q0 = __fmul_rn(x, y);
                const float r = fmaf(-q0, s, x);
                // s > 0, so the quotient has x's sign; the refinement alone would turn
                // x = -0 into +0 (r = +0 + -0), and fp8 keeps the sign of zero.
                t[i] = __builtin_amdgcn_fmed3f(copysignf(fmaf(r, y, q0), x), -448.0f, 448.0f);
            }
            int b = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
            b = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], b, true);
            w[j] = (uint32_t)b;
        }
        if constexpr (E == 8)
            *reinterpret_cast<u32x2*>(q) = u32x2{w[0], w[1]};
        else
            *reinterpret_cast<uint32_t*>(q) = w[0];
    }
    // Asymmetric codes; y = 1 / s correctly rounded, z the row's zero point.
    __device__ inline void store_codes_asym(int8_t* q, float s, float y, float z) const {
        uint32_t w[E / 4];
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
            uint32_t b = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b = code_u8_asym(v[4 * j + i], s, y, z, i, b);
            w[j] = b ^ 0x80808080u;
        }
        if constexpr (E == 8)
            *reinterpret_cast<u32x2*>(q) = u32x2{w[0], w[1]};
        else
            *reinterpret_cast<uint32_t*>(q) = w[0];
    }
    // y = 1 / s, correctly rounded.
    __device__ inline void store_codes(int8_t* q, float s, float y) const {
        uint32_t w[E / 4];
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
            uint32_t b = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b = code_u8_biased(v[4 * j + i], s, y, i, b);
            w[j] = b ^ 0x80808080u;   // code + 128 -> two's complement code
        }
        if constexpr (E == 8)
            *reinterpret_cast<u32x2*>(q) = u32x2{w[0], w[1]};
        else
            *reinterpret_cast<uint32_t*>(q) = w[0];
    }
};

// One workgroup per row. Rows of up to QT * QMAXC chunks stay in registers (one HBM
// read); longer rows are read a second time for the codes (the re-read hits L2).
// QMAXC is QC_SHORT or QC_LONG.
// E4M3: fp8 codes with s = max(absmax, 1e-10) / 448 (hotelren.com: the fp8 quantizer
// differs from the int8 one only in the result type; 448 is E4M3's largest value).
template <bool F16, bool E4M3, int QMAXC>
__global__ __launch_bounds__(QT) void quant_rows_i8_kernel(const void* __restrict__ x, int64_t K,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
    constexpr float QMAX = E4M3 ? 448.0f : 127.0f;
    auto codes = [&](const Chunk<F16>& c, int8_t* dst, float s, float y) {
        if constexpr (E4M3)
            c.store_codes_e4m3(reinterpret_cast<uint8_t*>(dst), s, y);
        else
            c.store_codes(dst, s, y);
    };
    using C = Chunk<F16>;
    __shared__ float red[QT / WAVE];
    const int64_t row = blockIdx.x;
    const char* xr = reinterpret_cast<const char*>(x) + row * K * (F16 ? 2 : 4);
    int8_t* qr = q + row * K;
    const int nch = (int)(K / C::E);

    float amax = 0.0f;
    if (nch <= QT * QMAXC) {
        C c[QMAXC];
#pragma unroll
        for (int i = 0; i < QMAXC; ++i) {
            const int ch = threadIdx.x + i * QT;
            if (ch < nch) {
                c[i].load(xr + (int64_t)ch * 16);
                amax = fmaxf(amax, c[i].absmax());
            }
        }
        amax = block_max(amax, red);
        const float s = fmaxf(amax, 1e-10f) / QMAX;
        const float y = 1.0f / s;
        if (threadIdx.x == 0)
            scale[row] = s;
#pragma unroll
        for (int i = 0; i < QMAXC; ++i) {
            const int ch = threadIdx.x + i * QT;
            if (ch < nch)
                codes(c[i], qr + (int64_t)ch * C::E, s, y);
        }
    } else {
        for (int ch = threadIdx.x; ch < nch; ch += QT) {
            C c;
            c.load(xr + (int64_t)ch * 16);
            amax = fmaxf(amax, c.absmax());
        }
        amax = block_max(amax, red);
        const float s = fmaxf(amax, 1e-10f) / QMAX;
        const float y = 1.0f / s;
        if (threadIdx.x == 0)
            scale[row] = s;
        for (int ch = threadIdx.x; ch < nch; ch += QT) {
            C c;
            c.load(xr + (int64_t)ch * 16);
            codes(c, qr + (int64_t)ch * C::E, s, y);
        }
    }
}

// Per-tensor symmetric int8 (hotelren.com "量化算法的本质", per_tensor_quant_int8: one scale
// for the whole array, s = max(absmax, 1e-10) / 127, codes as the per-row quantizer's). The
// caller's one-float scale output is the only accumulator, so three launches run in order on
// the stream: zero it; fold every workgroup's scale s_wg = max(absmax_wg, 1e-10) / 127 into it
// with one atomic max on the float's bits (non-negative floats order like their bit patterns,
// and a -> max(a, 1e-10) / 127, a correctly rounded division, never decreases, so the largest
// s_wg is exactly the s of the whole array's absmax); write the codes with that s.
constexpr int TCH = 4;   // 16-byte chunks per thread per step of the grid-stride loops

__global__ __launch_bounds__(64) void tensor_slot_zero_kernel(float* __restrict__ slot) {
    if (threadIdx.x == 0)
        *slot = 0.0f;
}

template <bool F16>
__global__ __launch_bounds__(QT) void tensor_absmax_kernel(const void* __restrict__ x, int64_t nch,
                                                           float* __restrict__ slot) {
    using C = Chunk<F16>;
    __shared__ float red[QT / WAVE];
    const char* xb = reinterpret_cast<const char*>(x);
    const int64_t stride = (int64_t)gridDim.x * QT * TCH;
    float amax = 0.0f;
    for (int64_t base = (int64_t)blockIdx.x * QT * TCH + threadIdx.x; base < nch; base += stride) {
        C c[TCH];
#pragma unroll
        for (int i = 0; i < TCH; ++i)
            if (base + i * QT < nch)
                c[i].load(xb + (base + i * QT) * 16);
#pragma unroll
        for (int i = 0; i < TCH; ++i)
            if (base + i * QT < nch)
                amax = fmaxf(amax, c[i].absmax());
    }
    amax = block_max(amax, red);
    // Device-scope atomics on one address serialize at the memory side, so most workgroups
    // skip theirs: the slot only grows, and a workgroup whose scale does not exceed the
    // value it reads (never more than the final one) cannot change the result.
    if (threadIdx.x == 0) {
        unsigned int* p = reinterpret_cast<unsigned int*>(slot);
        const unsigned int mine = __float_as_uint(fmaxf(amax, 1e-10f) / 127.0f);
        if (mine > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(p, mine);
    }
}

template <bool F16>
__global__ __launch_bounds__(QT) void tensor_codes_kernel(const void* __restrict__ x, int64_t nch,
                                                          const float* __restrict__ slot,
                                                          int8_t* __restrict__ q) {
    using C = Chunk<F16>;
    const char* xb = reinterpret_cast<const char*>(x);
    const float s = *slot;
    const float y = 1.0f / s;
    const int64_t stride = (int64_t)gridDim.x * QT * TCH;
    for (int64_t base = (int64_t)blockIdx.x * QT * TCH + threadIdx.x; base < nch; base += stride) {
        C c[TCH];
#pragma unroll
        for (int i = 0; i < TCH; ++i)
            if (base + i * QT < nch)
                c[i].load(xb + (base + i * QT) * 16);
#pragma unroll
        for (int i = 0; i < TCH; ++i)
            if (base + i * QT < nch)
                c[i].store_codes(q + (base + i * QT) * C::E, s, y);
    }
}

// Asymmetric per-row int8 (hotelren.com "量化算法的本质", per_channel_quant_int8, the
// asymmetric branch), per row with lo, hi its minimum and maximum:
//   s = max((hi - lo) / 255, 1e-8);  z = -lo / s - 128 (a float);
//   q = clamp(round(x / s + z), -128, 127)      (fp32, round half to even)
// so that x ~ s (q - z). One workgroup per row, as quant_rows_i8_kernel.
template <bool F16, int QMAXC>
__global__ __launch_bounds__(QT) void quant_rows_i8_asym_kernel(const void* __restrict__ x, int64_t K,
                                                               int8_t* __restrict__ q,
                                                               float* __restrict__ scale,
                                                               float* __restrict__ zero) {
    using C = Chunk<F16>;
    __shared__ float red[2 * (QT / WAVE)];
    const int64_t row = blockIdx.x;
    const char* xr = reinterpret_cast<const char*>(x) + row * K * (F16 ? 2 : 4);
    int8_t* qr = q + row * K;
    const int nch = (int)(K / C::E);
    float lo = INFINITY, hi = -INFINITY;
    auto params = [&](float& s, float& y, float& z) {
        block_minmax(lo, hi, red);
        s = fmaxf((hi - lo) / 255.0f, 1e-8f);
        y = 1.0f / s;
        z = __fsub_rn(-lo / s, 128.0f);
        if (threadIdx.x == 0) {
            scale[row] = s;
            zero[row] = z;
        }
    };
    float s, y, z;
    if (nch <= QT * QMAXC) {
        C c[QMAXC];
#pragma unroll
        for (int i = 0; i < QMAXC; ++i) {
            const int ch = threadIdx.x + i * QT;
            if (ch < nch) {
                c[i].load(xr + (int64_t)ch * 16);
                c[i].minmax(lo, hi);
            }
        }
        params(s, y, z);
#pragma unroll
        for (int i = 0; i < QMAXC; ++i) {
            const int ch = threadIdx.x + i * QT;
            if (ch < nch)
                c[i].store_codes_asym(qr + (int64_t)ch * C::E, s, y, z);
        }
    } else {
        for (int ch = threadIdx.x; ch < nch; ch += QT) {
            C c;
            c.load(xr + (int64_t)ch * 16);
            c.minmax(lo, hi);
        }
        params(s, y, z);
        for (int ch = threadIdx.x; ch < nch; ch += QT) {
            C c;
            c.load(xr + (int64_t)ch * 16);
            c.store_codes_asym(qr + (int64_t)ch * C::E, s, y, z);
        }
    }
}

// Column sums of int8 codes stored [N][K] (W column-major): the per-column term of the
// asymmetric expansion sum_k (q_x - z_x) q_w = sum_k q_x q_w - z_x sum_k q_w
// (quant67.com ch.17 §二). One workgroup per column; an offline producer.
__global__ __launch_bounds__(QT) void column_sums_i8_kernel(const int8_t* __restrict__ wq, int64_t K,
                                                           int32_t* __restrict__ colsum) {
    __shared__ int red[QT / WAVE];
    const int8_t* col = wq + (int64_t)blockIdx.x * K;
    int t = 0;
    for (int64_t c = threadIdx.x; c < K / 16; c += QT) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(col + c * 16);
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                t += (int)(int8_t)(v[d] >> (8 * b));
    }
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1)
        t += __shfl_xor(t, o, WAVE);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        red[threadIdx.x / WAVE] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        int r = 0;
#pragma unroll
        for (int i = 0; i < QT / WAVE; ++i)
            r += red[i];
        colsum[blockIdx.x] = r;
    }
}

// The weight producers give each (column, group) to a sub-group of LP lanes of one wave
// (LP the power of two at or above the group's chunk count, at most 64), so that a wave's
// loads are contiguous runs of the column: the lanes of a sub-group stride over the group's
// chunks, reduce with xor shuffles inside the sub-group (offsets below LP never leave it),
// and each writes its own code words. 64 / LP groups share a wave.
__device__ inline int producer_lanes(int chunks) {
    int lp = 1;
    while (lp < chunks && lp < WAVE)
        lp <<= 1;
    return lp;
}

// Block-asymmetric uint8 (zingnex.cn "从零实现大语言模型 INT8 量化", 核心量化流程 steps 1-2),
// per block b of `block` weights along K and column n:
//   s = max((max - min) / 255, 1e-8);  zp = clamp(rint(-min / s), 0, 255)
//   q = clamp(rint(w / s) + zp, 0, 255)          (fp32, IEEE division, half to even)
// A chunk is 4 weights (16 bytes in, one 32-bit word of codes out).
__global__ __launch_bounds__(256) void quant_block_asym_u8_kernel(
    const float* __restrict__ w, int64_t K, int64_t N, int64_t block, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint8_t* __restrict__ zp) {
    const int64_t G = K / block;
    const int ch = (int)(block / 4);
    const int lp = producer_lanes(ch);
    const int lane = threadIdx.x & (WAVE - 1), li = lane & (lp - 1);
    const int64_t id = ((int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE) * (WAVE / lp) + lane / lp;
    const bool live = id < N * G;
    const int64_t n = live ? id / G : 0, g = live ? id % G : 0;
    const float* v = w + n * K + g * block;
    float mn = INFINITY, mx = -INFINITY;
    if (live)
        for (int c = li; c < ch; c += lp) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(v + 4 * c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mn = fminf(mn, t[j]);
                mx = fmaxf(mx, t[j]);
            }
        }
    for (int o = lp / 2; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
    }
    if (!live)
        return;
    float s = (mx - mn) / 255.0f;
    s = fmaxf(s, 1e-8f);
    const float zf = fminf(fmaxf(rintf(-mn / s), 0.0f), 255.0f);
    const int z = (int)zf;
    // w / s through the block's correctly rounded reciprocal and an exact remainder, as in
    // code_u8_biased: the correctly rounded quotient at three operations
    // (tests/quotient_identity.c checks this over the producer's domain of blocks)
    const float y = 1.0f / s;
    uint8_t* qo = q + n * K + g * block;
    for (int c = li; c < ch; c += lp) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(v + 4 * c);
        uint32_t b = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float q0 = __fmul_rn(t[j], y);
            int cq = (int)rintf(fmaf(fmaf(-q0, s, t[j]), y, q0)) + z;
            cq = cq < 0 ? 0 : (cq > 255 ? 255 : cq);
            b |= (uint32_t)cq << (8 * j);
        }
        *reinterpret_cast<uint32_t*>(qo + 4 * c) = b;
    }
    if (li == 0) {
        scale[id] = s;
        zp[id] = (uint8_t)z;
    }
}

// Per-group symmetric int4 (xdnf.cn INT4/FP16 mixed GEMM on CANN TBE, §5.1: scale =
// absmax / 7, stored fp16 per §3.1): s16 = fp16(max(absmax, 7 * 2^-24) / 7) (round to
// nearest even); q = clamp(round(w / s16), -8, 7), packed eight per int32 along K with
// element k % 8 = j in bits [4j, 4j+3]. A chunk is 8 weights (32 bytes in, one word out).
__global__ __launch_bounds__(256) void quant_int4_group_kernel(
    const float* __restrict__ w, int64_t K, int64_t N, int64_t group, int32_t* __restrict__ packed,
    _Float16* __restrict__ scales) {
    const int64_t G = K / group;
    const int ch = (int)(group / 8);
    const int lp = producer_lanes(ch);
    const int lane = threadIdx.x & (WAVE - 1), li = lane & (lp - 1);
    const int64_t id = ((int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE) * (WAVE / lp) + lane / lp;
    const bool live = id < N * G;
    const int64_t n = live ? id / G : 0, g = live ? id % G : 0;
    const float* v = w + n * K + g * group;
    float a = 0.0f;
    if (live)
        for (int c = li; c < ch; c += lp) {
            const f32x4 t0 = *reinterpret_cast<const f32x4*>(v + 8 * c);
            const f32x4 t1 = *reinterpret_cast<const f32x4*>(v + 8 * c + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a = fmaxf(a, fmaxf(fabsf(t0[j]), fabsf(t1[j])));
        }
    for (int o = lp / 2; o > 0; o >>= 1)
        a = fmaxf(a, __shfl_xor(a, o, WAVE));
    if (!live)
        return;
    const float floor_a = 7.0f * 0x1p-24f;
    const _Float16 h = (_Float16)(fmaxf(a, floor_a) / 7.0f);
    const float s = (float)h;
    // x / s through the correctly rounded reciprocal and an exact remainder (the correctly
    // rounded quotient; tests/quotient_identity.c checks scales of any binary32 exponent in
    // [-100, 100] with |x / s| <= 128, which holds the fp16 scales here)
    const float y = 1.0f / s;
    int32_t* po = packed + n * (K / 8) + g * (group / 8);
    for (int c = li; c < ch; c += lp) {
        const f32x4 t0 = *reinterpret_cast<const f32x4*>(v + 8 * c);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(v + 8 * c + 4);
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = j < 4 ? t0[j] : t1[j - 4];
            const float q0 = __fmul_rn(x, y);
            const float r = fminf(fmaxf(rintf(fmaf(fmaf(-q0, s, x), y, q0)), -8.0f), 7.0f);
            word |= ((uint32_t)(int)r & 0xFu) << (4 * j);
        }
        po[c] = (int32_t)word;
    }
    if (li == 0)
        scales[id] = h;
}

}  // namespace

// Lanes per (column, group) in the producers, as producer_lanes computes it on the device.
inline int producer_lanes_host(int chunks) {
    int lp = 1;
    while (lp < chunks && lp < WAVE)
        lp <<= 1;
    return lp;
}

// The chunk count per thread for rows of K values: short rows keep the smaller count.
inline bool long_rows(int64_t K, int x_is_f16) { return K / (x_is_f16 ? 8 : 4) > (int64_t)QT * QC_SHORT; }

ql_status launch_quant_rows_i8(const void* x, int x_is_f16, int64_t rows, int64_t K, int8_t* q,
                               float* scale, hipStream_t stream) {
    if (rows == 0)
        return QL_OK;
    const dim3 grid((unsigned)rows), block(QT);
    const bool lg = long_rows(K, x_is_f16);
    if (x_is_f16) {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_kernel<true, false, QC_LONG>), grid, block, 0, stream, x, K, q, scale);
        else
            hipLaunchKernelGGL((quant_rows_i8_kernel<true, false, QC_SHORT>), grid, block, 0, stream, x, K, q, scale);
    } else {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_kernel<false, false, QC_LONG>), grid, block, 0, stream, x, K, q, scale);
        else
            hipLaunchKernelGGL((quant_rows_i8_kernel<false, false, QC_SHORT>), grid, block, 0, stream, x, K, q, scale);
    }
    return launch_status();
}

ql_status launch_quant_tensor_i8(const void* x, int x_is_f16, int64_t n, int8_t* q, float* scale,
                                 hipStream_t stream) {
    if (n == 0)
        return QL_OK;
    const int64_t nch = n / (x_is_f16 ? 8 : 4);
    const int64_t want = (nch + (int64_t)QT * TCH - 1) / ((int64_t)QT * TCH);
    const dim3 grid((unsigned)(want < 2048 ? want : 2048)), block(QT), one(1), w64(64);
    // the absmax pass uses at most two workgroups per CU: fewer atomics (see the kernel)
    const dim3 grid_max((unsigned)(want < 512 ? want : 512));
    hipLaunchKernelGGL(tensor_slot_zero_kernel, one, w64, 0, stream, scale);
    if (x_is_f16) {
        hipLaunchKernelGGL(tensor_absmax_kernel<true>, grid_max, block, 0, stream, x, nch, scale);
        hipLaunchKernelGGL(tensor_codes_kernel<true>, grid, block, 0, stream, x, nch, scale, q);
    } else {
        hipLaunchKernelGGL(tensor_absmax_kernel<false>, grid_max, block, 0, stream, x, nch, scale);
        hipLaunchKernelGGL(tensor_codes_kernel<false>, grid, block, 0, stream, x, nch, scale, q);
    }
    return launch_status();
}

ql_status launch_quant_rows_e4m3(const void* x, int x_is_f16, int64_t rows, int64_t K, uint8_t* q,
                                 float* scale, hipStream_t stream) {
    if (rows == 0)
        return QL_OK;
    const dim3 grid((unsigned)rows), block(QT);
    int8_t* qs = reinterpret_cast<int8_t*>(q);
    const bool lg = long_rows(K, x_is_f16);
    if (x_is_f16) {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_kernel<true, true, QC_LONG>), grid, block, 0, stream, x, K, qs, scale);
        else
            hipLaunchKernelGGL((quant_rows_i8_kernel<true, true, QC_SHORT>), grid, block, 0, stream, x, K, qs, scale);
    } else {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_kernel<false, true, QC_LONG>), grid, block, 0, stream, x, K, qs, scale);
        else
            hipLaunchKernelGGL((quant_rows_i8_kernel<false, true, QC_SHORT>), grid, block, 0, stream, x, K, qs, scale);
    }
    return launch_status();
}

ql_status launch_quant_rows_i8_asym(const void* x, int x_is_f16, int64_t rows, int64_t K, int8_t* q,
                                    float* scale, float* zero, hipStream_t stream) {
    if (rows == 0)
        return QL_OK;
    const dim3 grid((unsigned)rows), block(QT);
    const bool lg = long_rows(K, x_is_f16);
    if (x_is_f16) {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_asym_kernel<true, QC_LONG>), grid, block, 0, stream, x, K, q, scale, zero);
        else
            hipLaunchKernelGGL((quant_rows_i8_asym_kernel<true, QC_SHORT>), grid, block, 0, stream, x, K, q, scale, zero);
    } else {
        if (lg)
            hipLaunchKernelGGL((quant_rows_i8_asym_kernel<false, QC_LONG>), grid, block, 0, stream, x, K, q, scale, zero);
        else
            hipLaunchKernelGGL((quant_rows_i8_asym_kernel<false, QC_SHORT>), grid, block, 0, stream, x, K, q, scale, zero);
    }
    return launch_status();
}

ql_status launch_column_sums_i8(const int8_t* wq, int64_t K, int64_t N, int32_t* colsum,
                                hipStream_t stream) {
    if (N == 0)
        return QL_OK;
    hipLaunchKernelGGL(column_sums_i8_kernel, dim3((unsigned)N), dim3(QT), 0, stream, wq, K, colsum);
    return launch_status();
}

ql_status launch_quant_block_asym_u8(const float* w, int64_t K, int64_t N, int64_t block,
                                     uint8_t* q, float* scale, uint8_t* zp, hipStream_t stream) {
    const int64_t total = N * (K / block);
    if (total == 0)
        return QL_OK;
    const int64_t per_wg = (256 / WAVE) * (WAVE / producer_lanes_host((int)(block / 4)));
    const dim3 grid((unsigned)((total + per_wg - 1) / per_wg)), blk(256);
    hipLaunchKernelGGL(quant_block_asym_u8_kernel, grid, blk, 0, stream, w, K, N, block, q, scale,
                       zp);
    return launch_status();
}

ql_status launch_quant_int4_group(const float* w, int64_t K, int64_t N, int64_t group,
                                  int32_t* packed, void* scales, hipStream_t stream) {
    const int64_t total = N * (K / group);
    if (total == 0)
        return QL_OK;
    const int64_t per_wg = (256 / WAVE) * (WAVE / producer_lanes_host((int)(group / 8)));
    const dim3 grid((unsigned)((total + per_wg - 1) / per_wg)), blk(256);
    hipLaunchKernelGGL(quant_int4_group_kernel, grid, blk, 0, stream, w, K, N, group, packed,
                       reinterpret_cast<_Float16*>(scales));
    return launch_status();
}

}  // namespace ql
