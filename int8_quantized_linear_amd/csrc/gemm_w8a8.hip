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
// A workgroup of 8 waves (two per SIMD) computes a 256 x 256 output tile on
// v_mfma_i32_32x32x32_i8. K advances 128 bytes per stage through LDS buffers filled by
// direct buffer -> LDS copies (no register staging), whole 128-byte row pieces. The tile
// size is set by L2 -> CU bandwidth: a tile moves (BM + BN) bytes per k for BM * BN
// multiply-adds. The two 4-wave groups alternate between MFMA phases (with the copies
// spread between the MFMAs) and phases of LDS fragment reads, so a SIMD's MFMA stream
// never waits behind its own LDS reads. When the last round of 256 x 256 tiles would leave CUs idle, its N
// panels run as 128 x 256 or 128 x 192 tiles whose K is split between the two groups; a single
// partial round of big tiles runs as 256 x 192 tiles where those put more CUs to work; when
// no round of big tiles fills the chip, every tile is small, as 128 x 128 tiles where those
// make at most one round. K % 128 == 64 runs a last stage whose upper half reads zeros.
#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int NWAVES = 8;

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt immediate that waits until at most n vector-memory operations are pending
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// Workgroup barrier without a memory fence: __syncthreads() would also wait for every
// pending copy into LDS, including the stages still being prefetched. Each wave instead
// waits (vmcnt) for its own copies of the stage about to be read and (lgkmcnt) for its
// own LDS reads of the buffer about to be refilled, so after the barrier the stage is
// visible and the buffer is free. The "memory" clobber keeps the compiler from moving
// LDS accesses across the barrier.
__device__ inline void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// 4 bytes per lane from global memory straight into LDS (global_load_lds_dword): lane l's
// word lands at l * 4 past the wave-uniform LDS address.
__device__ inline void lds_copy4(const void* g, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 4, 0, 0);
#endif
}

// Bytes of the K ring at the start of the LDS allocation (three stages of a 128 x 256 tile
// with 128-byte k-steps); the tile's scales follow it: x_scale of its 256 rows, then
// w_scale and bias of its 256 columns, then (asymmetric activations only) x_zero of the
// rows and the code sums of the columns (4 bytes each); for int8 output the columns'
// output scales take the code sums' place.
constexpr int RING_BYTES = 3 * 384 * 128;
constexpr int SCALE_BYTES = 5 * 256 * 4;

// The epilogue's optional terms: for asymmetric activations the rows' zero points and W's
// column code sums (both NULL for symmetric activations); for int8 output the static output
// scales (out_scale_n of them: 1 for the whole output, or one per column).
struct EpiArgs {
    const float* x_zero;
    const int32_t* colsum;
    const float* out_scale;
    int out_scale_n;
};


// Operand element type: int8 codes (v_mfma_i32_32x32x32_i8, exact int32 sums) or OCP E4M3
// fp8 codes (v_mfma_f32_32x32x64_f8f6f4, fp32 sums). The bytes move the same way (copies,
// LDS layout and fragment reads are shared); one fp8 MFMA takes the two 16-byte fragments
// that two consecutive int8 substeps read, as the k order inside one MFMA is free as long as
// A and B agree.
enum { EL_I8 = 0, EL_E4M3 = 1 };
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
template <int ELEM>
using AccT = typename std::conditional<ELEM == EL_E4M3, f32x16, i32x16>::type;

// The bits of a scalar as another 32-bit type. Taking the value by copy matters: applied
// to a vector element (acc[i][j][e]) directly, __builtin_bit_cast reads element 0.
template <typename T, typename S>
__device__ __forceinline__ T bits_as(S s) {
    static_assert(sizeof(T) == sizeof(S), "same size");
    return __builtin_bit_cast(T, s);
}

__device__ inline i32x8 cat8(i32x4 lo, i32x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// The four 32-deep substeps of a 128-deep stage (F[ks][block]) into acc[i][j]. W's fragment
// is the matrix core's first operand and X's the second, so acc[i][j] holds the block
// transposed: element e of lane l is C[l & 31][8 (e >> 2) + 4 (l >> 5) + (e & 3)] of the
// 32 x 32 block (i, j). The products are the same either way; with this order the matrix
// cores draw less power on quantized activations (small codes) against weights (codes
// spread over the range), so the power-limited clock runs higher (measured A/B on one GPU:
// 57.8 -> 56.1 us at M = 2048, N = 8192, K = 4096).
template <int ELEM, int FM, int FN>
__device__ __forceinline__ void mfma_stage_of(AccT<ELEM> (&acc)[FM][FN], const i32x4 (&F)[4][FM + FN]) {
    if constexpr (ELEM == EL_I8) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F[ks][FM + j], F[ks][i], acc[i][j], 0, 0, 0);
    } else {
        // format 0 (E4M3) for A and B, no block scales
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        cat8(F[2 * kp][FM + j], F[2 * kp + 1][FM + j]), cat8(F[2 * kp][i], F[2 * kp + 1][i]),
                        acc[i][j], 0, 0, 0, 0, 0, 0);
    }
}

// f(activation, asymmetric) as compile-time constants for the launch's uniform choice: one
// epilogue instance per pair, so that none costs the others. The int32 output has neither.
template <int YMODE, typename F>
__device__ __forceinline__ void with_epilogue(int act, bool asym, F&& f) {
    using T = std::true_type;
    using U = std::false_type;
    if constexpr (YMODE == Y_I32) {
        f(std::integral_constant<int, ACT_NONE>{}, U{});
    } else if constexpr (YMODE == Y_I8) {
        if (act == ACT_GELU)
            f(std::integral_constant<int, ACT_GELU>{}, U{});
        else if (act == ACT_SILU)
            f(std::integral_constant<int, ACT_SILU>{}, U{});
        else
            f(std::integral_constant<int, ACT_NONE>{}, U{});
    } else if (asym) {
        if (act == ACT_GELU)
            f(std::integral_constant<int, ACT_GELU>{}, T{});
        else if (act == ACT_SILU)
            f(std::integral_constant<int, ACT_SILU>{}, T{});
        else
            f(std::integral_constant<int, ACT_NONE>{}, T{});
    } else {
        if (act == ACT_GELU)
            f(std::integral_constant<int, ACT_GELU>{}, U{});
        else if (act == ACT_SILU)
            f(std::integral_constant<int, ACT_SILU>{}, U{});
        else
            f(std::integral_constant<int, ACT_NONE>{}, U{});
    }
}

// Waves 0-3 each copy 64 of the tile's x_scale, w_scale and bias entries into LDS
// (indices clamped into range; entries past M or N are never used). Issued before the K
// loop's first copies, so every wait of the loop also covers them; the epilogue's barrier
// makes them visible to all waves. Without a bias, w_scale is copied in its place (unused).
__device__ inline void issue_scales(const float* xs, const float* ws, const float* bias, EpiArgs epi,
                                    int M, int N, int m0, int n0, int wave, int lane, int8_t* smem) {
    if (wave >= 4)
        return;
    int8_t* sc = smem + RING_BYTES + wave * 256;
    const int i = wave * 64 + lane;
    lds_copy4(xs + min(m0 + i, M - 1), sc);
    lds_copy4(ws + min(n0 + i, N - 1), sc + 1024);
    lds_copy4((bias != nullptr ? bias : ws) + min(n0 + i, N - 1), sc + 2048);
    if (epi.x_zero != nullptr) {
        lds_copy4(epi.x_zero + min(m0 + i, M - 1), sc + 3072);
        lds_copy4(epi.colsum + min(n0 + i, N - 1), sc + 4096);
    }
    if (epi.out_scale != nullptr)   // int8 output (never with zero points): the same slot
        lds_copy4(epi.out_scale + (epi.out_scale_n == 1 ? 0 : min(n0 + i, N - 1)), sc + 4096);
}

// Epilogue: the accumulators are dequantized (y = acc * x_scale[m] * w_scale[n] + bias[n])
// in registers and leave through LDS, one 32-row band of the wave's block at a time, so
// that global stores are whole 16-byte pieces of contiguous row segments rather than
// 2- or 4-byte scattered writes. Element e of block (i, j) in lane l is
// C[l & 31][8 (e >> 2) + 4 (l >> 5) + (e & 3)] of that 32 x 32 block (see mfma_stage_of):
// a lane holds one row and, for each g = e >> 2, four consecutive columns, which it stages
// with one store. Stores go through a buffer descriptor whose size ends at row M: the
// hardware drops stores of rows past M, and a column piece past N gets an offset beyond
// the size, so no store needs a branch.
// Workgroup barriers store_tile runs (a wave that does not store runs as many).
template <int YMODE>
constexpr int STORE_BARRIERS = YMODE == Y_I8 ? 2 : 1;

template <int WM, int WN, int FM, int FN, int YMODE, int NWV, int ACT, bool ASYM, typename ACC>
__device__ __forceinline__ void store_tile(const ACC (&acc)[FM][FN], bool has_bias,
                                           void* __restrict__ Y, int M, int N, int mrow0,
                                           int ncol0, int lm0, int ln0, int wave, int lane,
                                           int8_t* smem) {
    using OutT = typename std::conditional<YMODE == Y_F16, _Float16,
                 typename std::conditional<YMODE == Y_F32, float,
                 typename std::conditional<YMODE == Y_I8, int8_t, int32_t>::type>::type>::type;
    constexpr int SZ = sizeof(OutT);
    constexpr int VEC = 16 / SZ;                    // elements per 16-byte store
    // Staged row pitch: a row plus 16 bytes. A lane stages 4 * SZ bytes of its own row per
    // store, so the lanes served together sit in rows ROWB / 4 words apart: with the 16-byte
    // pad 16-byte stores (fp32, int32) hit distinct banks and 8-byte stores (fp16) at most two
    // to a bank (a 32-byte pad put four fp16 stores on one bank). Rows stay 16-byte aligned
    // for the 16-byte reads below.
    constexpr int ROWB = WN * SZ + 16;
    // The band is read back in segments of SEGW columns, whose 16-byte pieces divide a wave's
    // 64 lanes evenly: the whole row, or 32 columns when the row's pieces do not (WN = 96).
    constexpr int SEGW = 64 % (WN * SZ / 16) == 0 ? WN : 32;
    constexpr int NSEG = WN / SEGW;
    constexpr int LPR = SEGW * SZ / 16;             // lanes per staged row segment
    constexpr int RPI = 64 / LPR;                   // rows per read / store instruction
    constexpr int NRD = 32 / RPI;                   // reads (and stores) per band segment
    static_assert(WN % SEGW == 0 && 64 % LPR == 0, "segments tile the band");
    static_assert(NWV * 32 * ROWB <= RING_BYTES, "output staging fits the LDS ring");
    // Descriptor sizes are capped at LIM = 2^30 bytes, which no in-range offset reaches
    // (32 rows of at most 2^23 4-byte values); a column piece past N is sent to offset
    // row + LIM, at or past the size, and row + LIM stays below 2^31.
    constexpr int LIM = 1 << 30;
    using Out4 = OutT __attribute__((ext_vector_type(4)));

    barrier_no_fence();   // the ring is no longer read; every wave's scale copies landed
    int8_t* stage = smem + wave * 32 * ROWB;
    const float* sx = reinterpret_cast<const float*>(smem + RING_BYTES);
    const float* sw = sx + 256;
    const float* sb = sx + 512;
    const float* sz = sx + 768;
    const int32_t* scs = reinterpret_cast<const int32_t*>(sx + 1024);
    const int lr = lane & 31, lh = lane >> 5;
    // int8 output: the correctly rounded reciprocals of the tile's output scales, once per
    // tile, into the zero-point slot (int8 output has no zero points); y / s is then
    // q0 = RN(y r), RN(q0 + fma(-q0, s, y) r), the correctly rounded quotient. A second
    // barrier makes them visible (STORE_BARRIERS).
    if constexpr (YMODE == Y_I8) {
        float* srcp = const_cast<float*>(sz);
        for (int c = wave * 64 + lane; c < 256; c += NWV * 64)
            srcp[c] = 1.0f / reinterpret_cast<const float*>(scs)[c];
        __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0): the writes landed
        barrier_no_fence();
    }
    const bool vec_ok = (N % VEC) == 0;   // rows start 16-byte aligned
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        float xsv = 0.0f, zsv = 0.0f;
        if constexpr (YMODE != Y_I32) {
            xsv = sx[lm0 + 32 * i + lr];
            if constexpr (ASYM)
                zsv = sz[lm0 + 32 * i + lr];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = ln0 + 32 * j + 8 * g + 4 * lh;   // first of the four columns
                f32x4 wsv{}, bv{}, csv{}, osv{}, orv{};
                if constexpr (YMODE != Y_I32 && YMODE != Y_I8) {
                    wsv = *reinterpret_cast<const f32x4*>(sw + c0);
                    if (has_bias)
                        bv = *reinterpret_cast<const f32x4*>(sb + c0);
                    if constexpr (ASYM) {
                        const i32x4 cs = *reinterpret_cast<const i32x4*>(scs + c0);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            csv[q] = (float)cs[q];   // exact: |sum| <= 128 K < 2^24
                    }
                } else if constexpr (YMODE == Y_I8) {
                    wsv = *reinterpret_cast<const f32x4*>(sw + c0);
                    if (has_bias)
                        bv = *reinterpret_cast<const f32x4*>(sb + c0);
                    osv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(scs) + c0);
                    orv = *reinterpret_cast<const f32x4*>(sz + c0);
                }
                Out4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = 4 * g + q;
                    if constexpr (YMODE == Y_I32) {
                        v[q] = acc[i][j][e];
                    } else if constexpr (YMODE == Y_I8) {
                        v[q] = requant_code(activation<ACT>(epilogue_unfused((float)acc[i][j][e], xsv, wsv[q], bv[q])),
                                            osv[q], orv[q]);
                    } else if constexpr (ASYM) {
                        // sum_k (q_x - z_x) q_w = acc - z_x colsum, with one rounding
                        const float t = fmaf(-zsv, csv[q], (float)acc[i][j][e]);
                        v[q] = (OutT)activation<ACT, YMODE == Y_F16>(t * xsv * wsv[q] + bv[q]);
                    } else {
                        v[q] = (OutT)activation<ACT, YMODE == Y_F16>((float)acc[i][j][e] * xsv * wsv[q] + bv[q]);
                    }
                }
                *reinterpret_cast<Out4*>(stage + lr * ROWB + (32 * j + 8 * g + 4 * lh) * SZ) = v;
            }
        }
        // The wave's LDS operations complete in order, so its reads below see all of its
        // writes above; this only keeps the compiler from reordering them.
        asm volatile("" ::: "memory");
        const int row0 = mrow0 + 32 * i;
        const int64_t left = (int64_t)(M - row0) * N * SZ;   // bytes from row0 to the end
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<int8_t*>(Y) + (int64_t)row0 * N * SZ, 0,
            (int)(left <= 0 ? 0 : (left < LIM ? left : LIM)), 0x00020000);
        // Reads and stores go in batches of at most four 16-byte pieces per lane, which
        // keeps the band's registers few beside the accumulators.
        constexpr int PB = NRD < 4 ? NRD : 4;
#pragma unroll
        for (int sg = 0; sg < NSEG; ++sg) {
            // this lane's column in the segment, and the byte offset of its 16-byte piece in
            // the first row it stores
            const int cseg = sg * SEGW + (lane % LPR) * VEC;
            const int n = ncol0 + cseg;
            const int lane_off = (lane / LPR) * N * SZ + (n < N ? n * SZ : LIM);
#pragma unroll
            for (int p0 = 0; p0 < NRD; p0 += PB) {
                u32x4 rv[PB];
#pragma unroll
                for (int b = 0; b < PB; ++b) {
                    const int r = (p0 + b) * RPI + lane / LPR;
                    rv[b] = *reinterpret_cast<const u32x4*>(stage + r * ROWB + cseg * SZ);
                }
                if (vec_ok) {
#pragma unroll
                    for (int b = 0; b < PB; ++b)
                        __builtin_amdgcn_raw_buffer_store_b128(rv[b], rs, lane_off + (p0 + b) * RPI * N * SZ, 0, 0);
                } else {
#pragma unroll
                    for (int b = 0; b < PB; ++b) {
                        const int roff = ((p0 + b) * RPI + lane / LPR) * N * SZ;
                        const OutT* pv = reinterpret_cast<const OutT*>(&rv[b]);
#pragma unroll
                        for (int q = 0; q < VEC; ++q) {
                            const int off = roff + (n + q < N ? (n + q) * SZ : LIM);
                            if constexpr (SZ == 1)
                                __builtin_amdgcn_raw_buffer_store_b8(__builtin_bit_cast(uint8_t, pv[q]), rs, off, 0, 0);
                            else if constexpr (SZ == 2)
                                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, pv[q]), rs, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pv[q]), rs, off, 0, 0);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        asm volatile("" ::: "memory");   // the next band's writes follow these reads
    }
}

// Rows of 128 bytes (eight 16-byte chunks): chunk c of row r is stored at chunk position
// c ^ h128(r), which differs across any 8 consecutive rows and, with the row parity,
// across any 16, so the rows one fragment read touches fall in distinct bank groups.
__device__ inline int h128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l's
// bytes land at l * 16 past the wave-uniform LDS address. The per-lane offset is 32-bit
// and the wave-uniform part (the k-step) goes in the scalar offset. Device pass only.
__device__ inline void lds_copy16_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
#endif
}

// Vector offset of one lane's 16 bytes of a stage copy: v (the lane's row times K plus its
// chunk) + so (the k-step and the copy's 8-row step, wave-uniform). The row goes into the
// vector offset, so a row past the descriptor's end is out of range (the hardware returns
// zeros) whether or not the range check counts the scalar offset. `hi` (2^30 for a lane
// whose chunk lies in the upper half of the stage when K % 128 == 64, else 0) masked by
// `cutm` (all ones for the last stage) sends the lane out of range too: a half-deep last
// stage reads zeros above its 64 bytes. Offsets stay below 2^31.
__device__ inline int copy_voff(int v, int so, int hi, int cutm) { return (v + so) | (hi & cutm); }

// The wave-uniform part of a copy offset, opaque to the compiler: otherwise it splits off
// the loop-invariant 8-row step and keeps one hoisted vector offset per copy alive across
// the K loop, which costs registers the fragments need.
__device__ inline int stage_soff(int v) {
    asm volatile("" : "+s"(v));
    return v;
}

// A BM x BN tile on 8 waves with a ping-pong schedule. Waves 0-3
// (group 0) and 4-7 (group 1) put one wave of each group on every SIMD, and the two
// groups alternate between phases separated by workgroup barriers: in each phase one
// group issues nothing but the 32 MFMAs of a whole 128-deep stage (its fragments already
// in registers), while the other group reads the next stage's fragments from LDS and then
// issues its share of the copies. The MFMA stream of a SIMD never waits behind an LDS
// read or a copy of its own wave, and the copies' address work in the texture unit (16
// bytes a lane, one copy every ~16 clocks per CU) is split evenly between the two phases.
// Wave w owns the (BM / 2) x (BN / 4) block at rows (BM / 2) (w & 1), columns (BN / 4)
// (w >> 1); with BN = 192 (whose quarters are not whole 32-column blocks) the (BM / 4) x
// (BN / 2) block at rows (BM / 4) (w & 3), columns (BN / 2) (w >> 2). Either way group 0
// reads all of A and the low half of B's columns, group 1 all of A and the high half, so
// the three parts of a stage buffer (A, B low, B high) fall free at different times.
//
// Phase 2j (A_j):    group 0 runs stage j's MFMAs; group 1 reads stage j, then copies B
//                    high of stage j + 1 and B low of stage j + 2.
// Phase 2j+1 (B_j):  group 0 reads stage j + 1, then copies A of stage j + 2; group 1 runs
//                    stage j's MFMAs.
// Each part is refilled only after both of its reads are done (barriers between), and
// each wave waits for its copies at the end of its next (MFMA) phase, a phase before
// their first read.
template <int BM, int BN, int YMODE, int ELEM>
__device__ __forceinline__ void gemm_tile_pp(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                             const int8_t* __restrict__ B, const float* __restrict__ ws,
                                             const float* __restrict__ bias, void* __restrict__ Y,
                                             int M, int N, int K, int m0, int n0, int act, EpiArgs epi,
                                             int8_t* smem) {
    constexpr int BKL = 128;
    constexpr bool ROWS4 = BN % 128 != 0;   // four row blocks per group, two column halves
    constexpr int WM = ROWS4 ? BM / 4 : BM / 2, WN = ROWS4 ? BN / 2 : BN / 4, FM = WM / 32, FN = WN / 32;
    constexpr int STAGE_A = BM * BKL, STAGE = (BM + BN) * BKL;
    constexpr int CA = BM / 32, CH = BN / 64;   // per wave: copies of A, and of each half of B (8 rows each)
    static_assert(2 * STAGE <= RING_BYTES, "two stages fit the LDS allocation");
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0 && CA % 2 == 0 && BN % 64 == 0,
                  "tile shape");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm = ROWS4 ? wave & 3 : wave & 1, wn = ROWS4 ? wave >> 2 : wave >> 1;
    const int KT = (K + BKL - 1) / BKL;   // the last stage may be half deep (K % 128 == 64)

    // Wave q copies rows (BM / 4) q .. of A, and rows (BN / 8) q .. of each half of B: copy
    // c moves 8 rows x 128 bytes, lane l row R + 8 c + (l >> 3), logical chunk
    // (l & 7) ^ h128(row) (landing at chunk position l & 7). Rows past M or N read as zeros
    // (outside the descriptor).
    const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A) + (int64_t)m0 * K, 0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B) + (int64_t)n0 * K, 0, rows_b * K, 0x00020000);
    // Row R + 8 c + (l >> 3) (R a multiple of 8) has h128 = ((l >> 3) & 7) ^ ((R / 8 + c) & 1),
    // so a lane's offset is one of two values plus 8 c rows and the k-step. R / 8 is even for
    // A's rows and for B's when each wave's share of a half (BN / 8 rows) is a multiple of 16;
    // with BN = 192 (24 rows a wave) it has the wave's parity, q & 1 (the half's base, 96 h
    // rows, is a multiple of 16).
    const int cra = (BM / 4) * q + (lane >> 3), crb = (BN / 8) * q + (lane >> 3);
    const int bpar = (BN / 64) % 2 == 0 ? 0 : q & 1;
    const int cx = (lane & 7) ^ ((lane >> 3) & 7);
    const int va0 = cra * K + (cx << 4), va1 = cra * K + ((cx ^ 1) << 4);
    const int vb0 = crb * K + (cx << 4), vb1 = crb * K + ((cx ^ 1) << 4);
    // The lane's logical chunk is cx or cx ^ 1: in the upper half (k 64..127 of the stage)
    // exactly when cx >= 4. A half-deep last stage reads zeros there.
    const int hi = (K & (BKL - 1)) != 0 && cx >= 4 ? 0x40000000 : 0;
    // Copy c of A's rows, or of B's half h, of stage kt into buffer buf; see copy_voff.
    auto copy_a = [&](int kt, int buf, int c) {
        const int so = stage_soff(kt * BKL + 8 * c * K);
        lds_copy16_buf(ra, copy_voff((c & 1) ? va1 : va0, so, hi, kt == KT - 1 ? -1 : 0), 0,
                       smem + buf * STAGE + ((BM / 4) * q + 8 * c) * BKL);
    };
    auto copy_b = [&](int kt, int buf, int h, int c) {
        const int so = stage_soff(kt * BKL + (h * (BN / 2) + 8 * c) * K);
        lds_copy16_buf(rb, copy_voff(((c ^ bpar) & 1) ? vb1 : vb0, so, hi, kt == KT - 1 ? -1 : 0), 0,
                       smem + buf * STAGE + STAGE_A + (h * (BN / 2) + (BN / 8) * q + 8 * c) * BKL);
    };

    AccT<ELEM> acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // Fragments of a whole stage: F[ks][A blocks then B blocks], ks the 32-deep substep.
    const int lr = lane & 31;
    // Lane l reads row l & 31 of a 32-row block, logical chunk 2 ks + (l >> 5) of substep ks,
    // stored at chunk position (2 ks + (l >> 5)) ^ h128(row) = ((l >> 5) ^ h128(row)) ^ 2 ks:
    // substep ks flips bit 5 and 6 of the substep-0 offset. Stage and block bases are
    // multiples of 128, so they can be added before the flip.
    const int rbase = lr * BKL + (((lane >> 5) ^ h128(lr)) << 4);
    i32x4 F[4][FM + FN];
    auto read_stage = [&](int kt) {
        const int sbuf = (kt & 1) * STAGE;
        const int ta = rbase + stage_soff(sbuf + wm * WM * BKL);
        const int tb = rbase + stage_soff(sbuf + STAGE_A + wn * WN * BKL);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int8_t* pa = smem + (ta ^ (ks << 5));
            const int8_t* pb = smem + (tb ^ (ks << 5));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                F[ks][FM + j] = *reinterpret_cast<const i32x4*>(pb + j * 32 * BKL);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                F[ks][i] = *reinterpret_cast<const i32x4*>(pa + i * 32 * BKL);
        }
    };
    auto mfma_stage = [&]() { mfma_stage_of<ELEM, FM, FN>(acc, F); };

    // Prologue: group 0 copies all of stage 0 and stage 1 but its B high (copied in A_0),
    // and waits for stage 0; stage 1 has until the end of A_0.
    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, epi, M, N, m0, n0, wave, lane, smem);
    if (grp == 0) {
#pragma unroll
        for (int c = 0; c < CA; ++c)
            copy_a(0, 0, c);
#pragma unroll
        for (int c = 0; c < 2 * CH; ++c)
            copy_b(0, 0, c / CH, c % CH);
        if (KT > 1) {
#pragma unroll
            for (int c = 0; c < CA; ++c)
                copy_a(1, 1, c);
#pragma unroll
            for (int c = 0; c < CH; ++c)
                copy_b(1, 1, 0, c);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(CA + CH) & ~(0xF << 8));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_le(0) & ~(0xF << 8));
        }
    }
    barrier_no_fence();
    // Each group runs its own straight-line loops; both execute the same barriers in the
    // same order (two per stage). sched_barrier keeps the compiler from moving MFMAs (which
    // the barrier's memory clobber does not pin) from one phase into another. Stages near
    // the end have fewer copies; they run in loops of their own (a branch inside one loop
    // would make the compiler keep two sets of fragment registers).
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int LGKM0 = vmcnt_le(63) & ~(0xF << 8);   // lgkmcnt(0), vmcnt left alone
    // An MFMA phase: the stage's MFMAs, then this wave's copies (all issued in its reading
    // phase before) have landed.
    auto mfma_phase = [&]() {
        mfma_stage();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
        phase_end();
    };
    if (grp == 0) {
        read_stage(0);
        __builtin_amdgcn_s_waitcnt(LGKM0);
        phase_end();
        // A_j: MFMAs of stage j (in A_0 the prologue's stage 1 lands). B_j: reads of stage
        // j + 1 (past the end a repeat, never used), then the copies of A of stage j + 2.
        int j = 0;
        for (; j + 2 < KT; ++j) {
            mfma_phase();
            read_stage(j + 1);
#pragma unroll
            for (int c = 0; c < CA; ++c)
                copy_a(j + 2, j & 1, c);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(CA) & ~(0xF << 8));
            phase_end();
        }
        for (; j < KT; ++j) {
            mfma_phase();
            read_stage(min(j + 1, KT - 1));
            __builtin_amdgcn_s_waitcnt(LGKM0);
            phase_end();
        }
    } else {
        phase_end();   // while group 0 reads stage 0
        // A_j: reads of stage j, then the copies of B high of stage j + 1 and B low of stage
        // j + 2. B_j: MFMAs of stage j.
        int j = 0;
        for (; j + 2 < KT; ++j) {
            read_stage(j);
#pragma unroll
            for (int c = 0; c < CH; ++c)
                copy_b(j + 1, (j + 1) & 1, 1, c);
#pragma unroll
            for (int c = 0; c < CH; ++c)
                copy_b(j + 2, j & 1, 0, c);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * CH) & ~(0xF << 8));
            phase_end();
            mfma_phase();
        }
        for (; j + 1 < KT; ++j) {
            read_stage(j);
#pragma unroll
            for (int c = 0; c < CH; ++c)
                copy_b(j + 1, (j + 1) & 1, 1, c);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(CH) & ~(0xF << 8));
            phase_end();
            mfma_phase();
        }
        for (; j < KT; ++j) {
            read_stage(j);
            __builtin_amdgcn_s_waitcnt(LGKM0);
            phase_end();
            mfma_phase();
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    with_epilogue<YMODE>(act, epi.x_zero != nullptr, [&](auto act_c, auto asym_c) {
        store_tile<WM, WN, FM, FN, YMODE, 8, decltype(act_c)::value, decltype(asym_c)::value, AccT<ELEM>>(
            acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN, wm * WM, wn * WN, wave, lane, smem);
    });
}

// A 128 x 256 tile on 8 waves with K split between two groups. Group 0
// (waves 0-3) accumulates the even 128-deep stages and group 1 (waves 4-7) the odd ones,
// each over the whole tile with a 2 x 2 arrangement of 64 x 128 wave blocks, so one wave
// of each group sits on every SIMD. Stage j is computed in phase j: its group issues the
// stage's 32 MFMAs per wave (fragments already in registers) with the copies of stage
// j + 3 spread between them, while the other group reads stage j + 1's fragments from
// LDS. Three LDS buffers give the copies a phase to land before their stage is read. At the end group 1's int32 sums are added
// to group 0's through LDS (exact) and group 0 writes the tile.
template <int BN, int YMODE, int ELEM>
__device__ __forceinline__ void gemm_tile_ks(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                             const int8_t* __restrict__ B, const float* __restrict__ ws,
                                             const float* __restrict__ bias, void* __restrict__ Y,
                                             int M, int N, int K, int m0, int n0, int act, EpiArgs epi,
                                             int8_t* smem) {
    constexpr int BM = 128, BKL = 128;
    constexpr int WM = 64, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    static_assert(BN == 256 || BN == 192 || BN == 128, "128 x 256, 128 x 192 or 128 x 128 tiles");
    constexpr int STAGE_A = BM * BKL, STAGE = (BM + BN) * BKL;
    constexpr int CA = BM / 32, CB = BN / 32;   // copies of A and B per wave of a group (8 rows each)
    static_assert(3 * STAGE <= RING_BYTES, "three stages fit the LDS allocation");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm = q & 1, wn = q >> 1;
    const int KT = (K + BKL - 1) / BKL;   // the last stage may be half deep (K % 128 == 64)

    // Copies (either group, in its reading phase): wave q moves rows 32 q .. of A and
    // 64 q .. of B; copy c is 8 rows x 128 bytes, lane l row R q + 8 c + (l >> 3), whose
    // h128 is ((l >> 3) & 7) ^ (c & 1); the 8 c rows go with the k-step in the scalar
    // offset. Rows past M or N get an offset past the descriptor: zeros.
    const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A) + (int64_t)m0 * K, 0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B) + (int64_t)n0 * K, 0, rows_b * K, 0x00020000);
    const int cra = (BM / 4) * q + (lane >> 3), crb = (BN / 4) * q + (lane >> 3);
    const int cx = (lane & 7) ^ ((lane >> 3) & 7);
    const int va0 = cra * K + (cx << 4), va1 = cra * K + ((cx ^ 1) << 4);
    const int vb0 = crb * K + (cx << 4), vb1 = crb * K + ((cx ^ 1) << 4);
    const int hi = (K & (BKL - 1)) != 0 && cx >= 4 ? 0x40000000 : 0;   // upper half of a half-deep last stage
    // Copy c (< CA: of A, else of B) of stage kt (< KT) into buffer kt % 3; see copy_voff.
    auto copy_one = [&](int kt, int c) {
        int8_t* st = smem + (kt % 3) * STAGE;
        const int cutm = kt == KT - 1 ? -1 : 0;
        if (c < CA) {
            const int so = stage_soff(kt * BKL + 8 * c * K);
            lds_copy16_buf(ra, copy_voff((c & 1) ? va1 : va0, so, hi, cutm), 0,
                           st + ((BM / 4) * q + 8 * c) * BKL);
        } else {
            const int cb = c - CA;
            const int so = stage_soff(kt * BKL + 8 * cb * K);
            lds_copy16_buf(rb, copy_voff((cb & 1) ? vb1 : vb0, so, hi, cutm), 0,
                           st + STAGE_A + ((BN / 4) * q + 8 * cb) * BKL);
        }
    };
    auto copies = [&](int kt) {
#pragma unroll
        for (int c = 0; c < CA + CB; ++c)
            copy_one(kt, c);
    };

    AccT<ELEM> acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    const int lr = lane & 31;
    // Lane l reads row l & 31 of a 32-row block, logical chunk 2 ks + (l >> 5) of substep ks,
    // stored at chunk position (2 ks + (l >> 5)) ^ h128(row) = ((l >> 5) ^ h128(row)) ^ 2 ks:
    // substep ks flips bit 5 and 6 of the substep-0 offset. Stage and block bases are
    // multiples of 128, so they can be added before the flip.
    const int rbase = lr * BKL + (((lane >> 5) ^ h128(lr)) << 4);
    i32x4 F[4][FM + FN];
    auto read_stage = [&](int kt) {
        const int sbuf = (kt % 3) * STAGE;
        const int ta = rbase + stage_soff(sbuf + wm * WM * BKL);
        const int tb = rbase + stage_soff(sbuf + STAGE_A + wn * WN * BKL);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int8_t* pa = smem + (ta ^ (ks << 5));
            const int8_t* pb = smem + (tb ^ (ks << 5));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                F[ks][FM + j] = *reinterpret_cast<const i32x4*>(pb + j * 32 * BKL);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                F[ks][i] = *reinterpret_cast<const i32x4*>(pa + i * 32 * BKL);
        }
    };
    auto mfma_stage = [&]() { mfma_stage_of<ELEM, FM, FN>(acc, F); };
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int LGKM0 = vmcnt_le(63) & ~(0xF << 8);   // lgkmcnt(0), vmcnt left alone

    // Prologue: group 0 copies stages 0 and 2, group 1 stage 1 (stage 2 is needed in phase
    // 1, before any phase-0 copy could land); group 0 reads stage 0.
    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, epi, M, N, m0, n0, wave, lane, smem);
    if (grp == 0) {
        copies(0);
        if (KT > 2) {
            copies(2);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(CA + CB) & ~(0xF << 8));   // stage 0 landed
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_le(0) & ~(0xF << 8));
        }
    } else if (KT > 1) {
        copies(1);
    }
    phase_end();
    // Phase j: group (j & 1) runs stage j's MFMAs and nothing else; the other group reads
    // stage j + 1 and then issues the copies of stage j + 3 into stage j's buffer (read in
    // phase j - 1). Unlike the big tile, the copies go in the reading phase: a half tile's
    // stage is one phase, so copies spread between the MFMAs would stall the MFMA stream for
    // a larger share of it (measured: 4.6% slower K loop). At the end of a phase each wave
    // has every copy but the ones it just issued landed: those of its previous reading
    // phase, which feed the reads of the next phase (in phase 0, group 0's stage 2 from the
    // prologue). Every wave runs the same barriers (one per phase). Before phase 0 group 0
    // reads stage 0 while group 1 waits for its stage-1 copies.
    // Each group runs its own straight-line loop over pairs of phases (a branch per phase
    // inside one loop would make the compiler keep two copies of the fragments). Phases
    // near the end issue no copies; they run in loops of their own.
    auto mfma_phase = [&]() {
        mfma_stage();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
        phase_end();
    };
    auto read_phase = [&](int j) {
        read_stage(min(j + 1, KT - 1));   // past the end: a repeat, never used
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0) & ~(0xF << 8));
        phase_end();
    };
    auto read_phase_copying = [&](int j) {   // phase j with j + 3 < KT
        read_stage(j + 1);
        copies(j + 3);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(CA + CB) & ~(0xF << 8));
        phase_end();
    };
    if (grp == 0) {
        read_stage(0);
        __builtin_amdgcn_s_waitcnt(LGKM0);
        phase_end();
        int j = 0;
        for (; j + 4 < KT; j += 2) {
            mfma_phase();                  // phase j
            read_phase_copying(j + 1);     // phase j + 1
        }
        for (; j + 1 < KT; j += 2) {
            mfma_phase();
            read_phase(j + 1);
        }
        if (j < KT)
            mfma_phase();
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));   // stage 1 landed
        phase_end();
        if (KT > 3)                        // phase 0
            read_phase_copying(0);
        else
            read_phase(0);
        int j = 1;
        for (; j + 4 < KT; j += 2) {
            mfma_phase();                  // phase j
            read_phase_copying(j + 1);     // phase j + 1
        }
        for (; j + 1 < KT; j += 2) {
            mfma_phase();
            read_phase(j + 1);
        }
        if (j < KT)
            mfma_phase();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));

    // Group 1's sums go to LDS (64 lanes x 16 ints per block, one block per 4 KB), then
    // group 0 adds them; the ring is free (every copy has landed, every read is done).
    phase_end();
    int32_t* xch = reinterpret_cast<int32_t*>(smem) + q * (FM * FN * 1024);
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    *reinterpret_cast<i32x4*>(xch + ((i * FN + j) * 4 + e4) * 256 + lane * 4) =
                        i32x4{bits_as<int32_t>(acc[i][j][4 * e4]), bits_as<int32_t>(acc[i][j][4 * e4 + 1]),
                              bits_as<int32_t>(acc[i][j][4 * e4 + 2]), bits_as<int32_t>(acc[i][j][4 * e4 + 3])};
    }
    phase_end();
    if (grp == 0) {
        // One block (16 ints a lane) at a time, each sum formed here (the empty asm keeps
        // the compiler from sinking the adds into the epilogue), so that group 1's sums
        // never all sit in registers beside the accumulators.
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const i32x4 v = *reinterpret_cast<const i32x4*>(xch + ((i * FN + j) * 4 + e4) * 256 + lane * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        using E = decltype(acc[i][j][0] + 0);
                        E sum = acc[i][j][4 * e4 + r] + bits_as<E>(v[r]);
                        asm volatile("" : "+v"(sum));
                        acc[i][j][4 * e4 + r] = sum;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    __builtin_amdgcn_s_waitcnt(LGKM0);
    if (grp == 0) {
        with_epilogue<YMODE>(act, epi.x_zero != nullptr, [&](auto act_c, auto asym_c) {
            store_tile<WM, WN, FM, FN, YMODE, 4, decltype(act_c)::value, decltype(asym_c)::value, AccT<ELEM>>(
                acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN, wm * WM, wn * WN, q, lane, smem);
        });
    } else {
#pragma unroll
        for (int b = 0; b < STORE_BARRIERS<YMODE>; ++b)
            barrier_no_fence();   // the barriers store_tile runs
    }
}

// Tiles: `nbig` 256 x BNB tiles (BNB = 256, or 192 when the big tiles make one partial round
// and nothing else) cover the first `nbig / tiles_m` N-panels and `nsmall` 128 x BNS tiles
// (BNS = 256, 192, or 128 when every tile is small) the remaining columns; workgroup b takes
// big tile b, then small tile b (or the small tile first, when staggered).
// With 256 CUs, whole rounds of big tiles keep every CU busy and the leftover panels run
// as half-height tiles in a shorter final round. Within each kind, tiles are dealt to
// XCDs so that an XCD's tiles are consecutive and share W panels (column-major order).
// `stagger` != 0: the workgroups b < nsmall with (b & stagger) != 0 run their half tile first
// and their big tile after it (below).
struct TilePlan {
    int tiles_m_big, nbig, tiles_m_small, nsmall, n_small0, bn_small, bn_big, stagger;
};

template <int YMODE, int ELEM, int BNS, int BNB>
__global__ __launch_bounds__(64 * NWAVES, 1) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int K, int act, EpiArgs epi, TilePlan plan) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[RING_BYTES + SCALE_BYTES];
    const int bid = blockIdx.x;
    // Staggered order: when every CU runs one big tile and then a half tile, all big tiles
    // finish together and their epilogues store the whole big-tile output (32 MiB at the
    // 2048 x 11008 layer) at once, with the matrix cores idle everywhere. Half of each XCD's
    // workgroups (bit 3 of b: workgroups are dealt to the XCDs round-robin) instead run the
    // half tile first, so half of that burst overlaps the other workgroups' K loops. The
    // tiles and their sums are unchanged.
    if ((bid & plan.stagger) != 0 && bid < plan.nsmall && bid < plan.nbig) {
        {
            const int tile = xcd_remap(bid, plan.nsmall);
            const int tn = tile / plan.tiles_m_small, tm = tile - tn * plan.tiles_m_small;
            gemm_tile_ks<BNS, YMODE, ELEM>(A, xs, B, ws, bias, Y, M, N, K, tm * 128, plan.n_small0 + tn * BNS, act,
                                          epi, smem);
        }
        // the half tile's epilogue has read all it needs from LDS
        __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0)
        barrier_no_fence();
        const int tile = xcd_remap(bid, plan.nbig);
        const int tn = tile / plan.tiles_m_big, tm = tile - tn * plan.tiles_m_big;
        gemm_tile_pp<256, BNB, YMODE, ELEM>(A, xs, B, ws, bias, Y, M, N, K, tm * 256, tn * BNB, act, epi, smem);
        return;
    }
    if (bid < plan.nbig) {
        const int tile = xcd_remap(bid, plan.nbig);
        const int tn = tile / plan.tiles_m_big, tm = tile - tn * plan.tiles_m_big;
        gemm_tile_pp<256, BNB, YMODE, ELEM>(A, xs, B, ws, bias, Y, M, N, K, tm * 256, tn * BNB, act, epi, smem);
        if (bid >= plan.nsmall)
            return;
        // The big tile's epilogue has read all it needs from LDS (its stores may still be in
        // flight): the half tile may refill the LDS.
        __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0)
        barrier_no_fence();
    }
    if (bid < plan.nsmall) {
        const int tile = xcd_remap(bid, plan.nsmall);
        const int tn = tile / plan.tiles_m_small, tm = tile - tn * plan.tiles_m_small;
        gemm_tile_ks<BNS, YMODE, ELEM>(A, xs, B, ws, bias, Y, M, N, K, tm * 128, plan.n_small0 + tn * BNS, act, epi,
                                      smem);
    }
}

TilePlan plan_tiles(int64_t M, int64_t N) {
    TilePlan p{};
    const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
    const int total = tm * tn, cus = cu_count();
    int small_panels = 0;
    if (M <= 128 || 2 * total <= cus) {
        // every tile is half height: with at most half the CUs' worth of big tiles, half
        // tiles (K split between the two wave groups) put twice as many CUs to work
        small_panels = tn;
    } else if (total > cus) {
        const int left = total % cus;           // tiles of the last, partial round
        if (left > 0 && left <= cus / 2)
            small_panels = (left + tm - 1) / tm;
    }
    p.tiles_m_big = tm;
    p.nbig = (tn - small_panels) * tm;
    p.tiles_m_small = (int)((M + 127) / 128);
    p.nsmall = small_panels * p.tiles_m_small;
    p.n_small0 = (tn - small_panels) * 256;
    p.bn_small = 256;
    p.bn_big = 256;
    return p;
}

// 256 x 192 big tiles when the 256 x 256 ones make one partial round and no small tiles follow
// (between half and all of the CUs), and the narrower tiles put more CUs to work, still in one
// round: each does three quarters of a big tile's work. Measured at K = 4096 (us, 256 x 256 /
// 256 x 192; the same int32 sums and outputs): M = 768, N = 11008 (129 / 174 tiles) 43.5 /
// 36.9; M = 1024, N = 11008 46.0 / 43.1; M = 768, N = 14336 44.9 / 42.1; M = 1280, N = 8192
// 43.8 / 40.4; M = 768, N = 11008, K = 11008 95.9 / 85.4.
int big_tiles_192(const TilePlan& p, int64_t N) { return p.tiles_m_big * (int)((N + 191) / 192); }

bool use_big_192(const TilePlan& p, int64_t N) {
    const int n = big_tiles_192(p, N);
    return p.nsmall == 0 && p.nbig > 0 && p.nbig < cu_count() && n > p.nbig && n <= cu_count();
}

TilePlan plan_big_192(TilePlan p, int64_t N) {
    p.nbig = big_tiles_192(p, N);
    p.bn_big = 192;
    return p;
}

// The 64 x 64 kernel (gemm_w8a8_mid.hip) takes the shapes where the tile plan puts at most
// half of the CUs to work and its own tiles make at most two rounds. Measured at K = 4096
// (us, tile plan against 64 x 64 tiles): N = 4096: M = 256 24.3 / 13.5, M = 512 25.5 / 17.2,
// M = 768 27.3 / 28.4; N = 11008: M = 129 26.7 / 27.0, M = 256 27.6 / 29.1; at M = 256,
// N = 4096 also K = 11008 53.7 / 30.6 and K = 14336 66.4 / 38.4.
// 128 x 128 small tiles instead of 128 x 256 when every tile is small and the 128 x 128 tiles
// make at most one round: twice the workgroups on the same two-group split-K schedule.
// Measured at K = 4096 (us, 128 x 256 / 128 x 128): N = 4096: M = 600 30.4 / 21.9, M = 768
// 31.5 / 23.0, M = 1024 31.2 / 23.1; N = 11008: M = 129 29.4 / 21.5, M = 256 34.0 / 24.1;
// N = 14336, M = 256 35.1 / 25.6; N = 4096, M = 1024, K = 11008 74.1 / 53.4; M = 768,
// K = 14336 92.7 / 65.9. Past one round it loses (M = 1536, N = 4096: 32.4 / 43.3; M = 384,
// N = 11008, 258 tiles: 32.6 / 34.6).
bool use_quarter_tiles(const TilePlan& p, int64_t N) {
    return p.nbig == 0 && (int64_t)p.tiles_m_small * ((N + 127) / 128) <= cu_count();
}

TilePlan quarter_plan(TilePlan p, int64_t N) {
    p.nsmall = p.tiles_m_small * (int)((N + 127) / 128);
    p.bn_small = 128;
    return p;
}

// Small tiles 192 columns wide where they make more workgroups than 256-wide ones and still
// at most one round: the small tiles run together, so the widest sets their time, and a CU's
// operand bytes per tile fall by a sixth. Measured at K = 4096 (us, 128 x 256 / 128 x 192; the
// same int32 sums and outputs): M = 2048, N = 11008 (256 big tiles, then 176 / 240 small)
// 86.6 / 84.0; M = 384, N = 11008 27.9 / 24.3; M = 512, N = 11008 30.6 / 27.4; M = 384,
// N = 14336 31.2 / 27.2; M = 600, N = 9000 30.8 / 27.6; M = 1025, N = 4096 28.6 / 24.7;
// M = 1536, N = 11008 78.6 / 74.4; M = 3072, N = 11008 132.9 / 128.2; M = 512, N = 11008,
// K = 11008 66.2 / 60.2.
int small_tiles_192(const TilePlan& p, int64_t N) {
    return p.tiles_m_small * (int)((N - p.n_small0 + 191) / 192);
}

bool use_192_tiles(const TilePlan& p, int64_t N) {
    const int n = small_tiles_192(p, N);
    return p.nsmall > 0 && n > p.nsmall && n <= cu_count();
}

TilePlan plan_192(TilePlan p, int64_t N) {
    p.nsmall = small_tiles_192(p, N);
    p.bn_small = 192;
    return p;
}

bool use_mid_tiles(const TilePlan& p, int64_t M, int64_t N) {
    const int wgs = p.nbig > p.nsmall ? p.nbig : p.nsmall;
    const int64_t mid = ((M + 63) / 64) * ((N + 63) / 64);
    return 2 * wgs <= cu_count() && mid <= 2 * (int64_t)cu_count();
}

}  // namespace

ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode, int act,
                           const float* x_zero, const int32_t* colsum, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream, bool e4m3, const float* out_scale,
                           int out_scale_n) {
    if (M == 0 || N == 0)
        return QL_OK;
    TilePlan plan = plan_tiles(M, N);
    if (use_mid_tiles(plan, M, N)) {
        // the tile plan would leave most CUs idle: 64 x 64 tiles instead
        return launch_gemm_w8a8_mid(xq, x_scale, wq, w_scale, bias, y, y_mode, act, x_zero, colsum, out_scale,
                                    out_scale_n, M, N, K, stream, e4m3);
    }
    if (use_quarter_tiles(plan, N))
        plan = quarter_plan(plan, N);
    else if (use_192_tiles(plan, N))
        plan = plan_192(plan, N);
    else if (use_big_192(plan, N))
        plan = plan_big_192(plan, N);
    // One round of big tiles followed by half tiles on the same workgroups: stagger the order
    // on half of them. Measured at K = 4096 (us, all big-first / staggered; the same outputs):
    // M = 2048, N = 11008 83.1 / 80.6 and 82.9 / 80.3; N = 10000 82.4 / 81.4; N = 8704 76.7 /
    // 74.7; M = 1792, N = 11008 81.6 / 81.1; M = 2048, N = 9000 77.2 / 77.5; at K = 11008
    // 192.5 / 191.0. With two rounds of big tiles (M = 3072, N = 11008) staggering delayed the
    // first round (123.8 / 124.9), so it is not used there.
    plan.stagger = plan.nsmall > 0 && plan.nbig <= cu_count() ? 8 : 0;
    // Workgroup b runs big tile b (b < nbig) and then half tile b (b < nsmall), or the two the
    // other way round when staggered, so the half tiles need no dispatch of their own and
    // each tile's first copies overlap the previous tile's last stores.
    const dim3 grid((unsigned)(plan.nbig > plan.nsmall ? plan.nbig : plan.nsmall)), block(64 * NWAVES);
    const int m = (int)M, n = (int)N, k = (int)K;
#define QL_LAUNCH_ONE(MODE, EL, BNS, BNB)                                                                \
    hipLaunchKernelGGL((gemm_w8a8_kernel<MODE, EL, BNS, BNB>), grid, block, 0, stream, xq, x_scale, wq, w_scale, \
                       bias, y, m, n, k, act, (EpiArgs{x_zero, colsum, out_scale, out_scale_n}), plan)
#define QL_LAUNCH(MODE, EL)                                                                              \
    do {                                                                                                 \
        if (plan.bn_big == 192)                                                                          \
            QL_LAUNCH_ONE(MODE, EL, 256, 192);                                                           \
        else if (plan.bn_small == 128)                                                                   \
            QL_LAUNCH_ONE(MODE, EL, 128, 256);                                                           \
        else if (plan.bn_small == 192)                                                                   \
            QL_LAUNCH_ONE(MODE, EL, 192, 256);                                                           \
        else                                                                                             \
            QL_LAUNCH_ONE(MODE, EL, 256, 256);                                                           \
    } while (0)
    if (e4m3) {
        if (y_mode == Y_F32)
            QL_LAUNCH(Y_F32, EL_E4M3);
        else
            QL_LAUNCH(Y_F16, EL_E4M3);
        return launch_status();
    }
    switch (y_mode) {
    case Y_I8:
        QL_LAUNCH(Y_I8, EL_I8);
        break;
    case Y_F32:
        QL_LAUNCH(Y_F32, EL_I8);
        break;
    case Y_F16:
        QL_LAUNCH(Y_F16, EL_I8);
        break;
    default:
        QL_LAUNCH(Y_I32, EL_I8);
        break;
    }
#undef QL_LAUNCH
#undef QL_LAUNCH_ONE
    return launch_status();
}

}  // namespace ql
