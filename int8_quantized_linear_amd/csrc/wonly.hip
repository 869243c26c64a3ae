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
// of D k-steps of loads in flight, issued D steps ahead of use, and the columns are
// spread so that every CU gets a share (a workgroup covers ceil(N / CUs) columns, rounded
// up to 8; its 4 waves split K four ways).
//
// Every global load is laid out so that the four lanes of a quad read one contiguous
// piece: the L1 then serves a quad with one request, where four lanes on four rows or
// columns (the MFMA operand layout) cost four, which caps a CU at about a third of the
// rate. Weights come into registers that way and a lane permute puts them in MFMA order;
// activations are copied straight into a ring in LDS (16 bytes a lane, whole row pieces)
// and read back in MFMA order.
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
#include <type_traits>
#include <utility>

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

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// The same with the subtraction written on fp16 pairs, `sub` already in both halves of
// sub2: one v_pk_add_f16 per pair also when `sub` is not a constant. (For a run-time `sub`,
// the fp16x8 form above compiles to a subtraction per half and a repack, three instructions
// per pair.) The zero-point format uses this form with 64-column workgroups, where it
// measured 6-7% faster; with 16 or 32 columns the other form's schedule measured 1-2% faster.
__device__ inline void bytes_to_f16_pairs(const u32x4 w, uint32_t flip, f16x2 sub2, f16x8& lo, f16x8& hi) {
    f16x2 p[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t v = w[d] ^ flip;
        p[2 * d] = __builtin_bit_cast(f16x2, magic_lo(v)) - sub2;
        p[2 * d + 1] = __builtin_bit_cast(f16x2, magic_hi(v)) - sub2;
    }
    lo = f16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
    hi = f16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

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

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at l * 16 past
// the wave-uniform LDS address. An offset past the descriptor's size writes zeros.
__device__ inline void lds_copy16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
#endif
}

template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order.
template <int N, typename F>
__device__ inline void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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

// Activation ring in LDS. A slot holds one k-step of the launch's XR rows (16 MT, or 8 for a
// launch of at most 8 rows, which then copies half as many bytes per step: W8A16 at M = 1
// 5.59 -> 5.30 us, block-asymmetric at M = 8 7.65 -> 7.35 us, measured A/B): RB bytes per
// row, filled by NXC copies of 1 KiB (RPC rows each). Chunk c (16 bytes) of row r sits at
// position c ^ (r & XM) of its row, so that the 16 lanes of an MFMA-layout read (16 rows,
// one chunk) fall on 16 different bank groups, while the 4 lanes of a copy quad still read
// one aligned 64-byte piece. With 8 rows per copy (128-byte rows) a 16-byte pad after each
// copy moves rows 8..15 to the other bank groups.
template <int KS, int XR>
struct XRing {
    static constexpr int RB = KS * 2;
    static constexpr int CPR = RB / 16;               // chunks per row
    static constexpr int RPC = 1024 / RB;             // rows per copy
    static constexpr int XM = CPR - 1;                // swizzle mask
    static constexpr int PAD = RPC == 8 ? 16 : 0;
    static constexpr int CSTRIDE = 1024 + PAD;        // bytes per copy in LDS
    static constexpr int NXC = XR / RPC;              // copies per slot
    static constexpr int SLOT = NXC * CSTRIDE;
    static constexpr int ISTRIDE = (16 / RPC) * CSTRIDE;   // bytes between 16-row blocks
    static constexpr int QV = CPR / RPC > 1 ? CPR / RPC : 1;   // copies before the swizzle repeats
    static constexpr int QROWS = QV * RPC;
};

// Waves per workgroup: two per SIMD at 17..32 rows, where each step carries enough work
// (dequantization and MFMAs) that a second wave per SIMD hides one wave's waits; one per
// SIMD otherwise, leaving LDS to deeper rings.
template <int MT>
constexpr int nwaves() { return MT == 2 ? 8 : 4; }
constexpr int LDS_BUDGET = 150 * 1024;  // activation rings + partial sums + scales

// Scales (and zero points) of the workgroup's columns, staged in LDS when they fit: 32 KB
// where the activation ring leaves room (one or three blocks of 16 rows, or two with
// 64-column tiles, which keep a single step in flight), else 16 KB. With 32 KB, 56 columns of 64 fp32
// scales and 64 zero points (N = 14336 over 256 CUs, K = 4096) fit: block-asymmetric at
// one row 24.4 -> 15.7 us, at 32 rows 27.3 -> 19.6 us, N = 28672 47.9 -> 27.6 us, against
// loading them from global memory every step. int4 keeps 16 KB beyond one row block (its fp16
// scales fit there, and the larger area measured 2% slower at 17..32 rows).
constexpr int sl_words(int fmt, int mt, int nt) {
    return mt == 1 || (fmt != W_INT4_SYM && (mt == 3 || (mt == 2 && nt == 4))) ? 8192 : 4096;
}

// Ring depth: k-steps in flight per wave, as a power of two (at most 8) so that it divides a
// wave's step count when K is a multiple of 4 * KS * D (the loop is padded to whole rings
// with zero-filled steps), and at least 2, or 1 for group scales with two waves per SIMD
// (where the other wave runs while one waits: int4 at 32 rows, N = 14336, 13.9 -> 13.1 us,
// N = 28672 26.6 -> 24.0 us, block-asymmetric 57.5 -> 55.4 us against a floor of 2; per-
// channel int8 there, and anything with one wave per SIMD, is slower with a single step). Bounded by the weight registers (about 280 per lane beside the
// accumulators and the operands of the step being computed), by the LDS activation ring,
// and by a budget of about 32K weights in flight per CU. More than that is slower: with a
// whole K range issued at once (a CU's 56 columns of 4096 int4 weights, say), the requests
// of every CU queue together, a wave's first step completes about when its last does, and
// none of the dequantization overlaps the transfer. Measured on MI355X, K = 4096, one row
// (event-timed bursts over cold weights), against depths set by registers and LDS alone:
// N = 14336 int4 12.9 -> 9.7 us, int8 15.0 -> 13.4 us; N = 28672 int4 24.6 -> 16.1 us;
// block-asymmetric N = 11008 19.1 -> 16.0 us; N = 4096 int4 at 16 rows 6.6 -> 5.9 us. From
// 17 rows on the LDS ring already held the depth at 2 (no change).
// The waves' partial sums share the first ring slot when they fit in it.
constexpr int INFLIGHT_WEIGHTS = 32768;   // per CU
// Rows of the activation ring: 16 per block, or 8 when the launch has at most 8 rows (HX).
template <int MT, bool HX>
constexpr int xrows() { return HX ? 8 : 16 * MT; }

template <int KS, int MT, int NT, bool HX>
constexpr int red_extra() {
    constexpr int red = nwaves<MT>() * MT * NT * 64 * 16, slot = nwaves<MT>() * XRing<KS, xrows<MT, HX>()>::SLOT;
    return red > slot ? red : 0;
}

template <int FMT, int KS, int MT, int NT, int SCALES, bool HX>
constexpr int ring_depth() {
    constexpr bool GLOAD = SCALES == 2;
    using G = Geo<FMT, KS>;
    constexpr int per_step = NT * (G::WB / 4) + (GLOAD ? NT * (FMT == W_UINT8_ZP ? 2 : 1) : 0);
    constexpr int fixed = MT * NT * 4 + 2 * MT * G::HN * 4 + 12 + NT * 2 + MT + 24 + G::HN;
    // one wave per SIMD may use about 280 registers (VGPRs and AGPRs); two share the file
    // and get about 200 each
    constexpr int dr = ((nwaves<MT>() == 4 ? 280 : 200) - fixed) / per_step;
    constexpr int dl = (LDS_BUDGET - sl_words(FMT, MT, NT) * 4 - red_extra<KS, MT, NT, HX>()) /
                       (nwaves<MT>() * XRing<KS, xrows<MT, HX>()>::SLOT);
    constexpr int db = INFLIGHT_WEIGHTS / (nwaves<MT>() * NT * 16 * KS);
    constexpr int d0 = dr < dl ? dr : dl;
    constexpr int d = d0 < db ? d0 : db;
    // at most 8: each slot is its own LDS array (see the kernel)
    return d >= 8 ? 8 : d >= 4 ? 4 : d >= 2 || nwaves<MT>() == 4 || SCALES == 0 ? 2 : 1;
}

// One workgroup of NW waves: `cols` (<= 16 NT) consecutive columns from col0, all M
// (<= 16 MT) rows. Wave w runs k-steps [s0, s1) (its 1/NW of K); lane (ln, lg) = (l & 15, l >> 4) handles
// column col0 + 16 j + ln of block j. SCALES: 0 = one scale per column (applied at the
// end), 1 = per group, staged in LDS, 2 = per group, loaded from global memory each step
// (blocks too large for LDS).
template <int FMT, int KS, int MT, int NT, int SCALES, int D, bool HX>
__global__ __launch_bounds__(64 * nwaves<MT>()) void wonly_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wc, const void* __restrict__ scale,
    const uint8_t* __restrict__ zp, int group, const float* __restrict__ bias,
    _Float16* __restrict__ Y, int M, int N, int K, int cols, int act) {
    using G = Geo<FMT, KS>;
    using XG = XRing<KS, xrows<MT, HX>()>;
    using WR = typename G::WR;
    constexpr int NW = nwaves<MT>();
    constexpr int HN = G::HN;
    constexpr bool GROUPED = SCALES != 0;
    constexpr bool ZP = FMT == W_UINT8_ZP;
    constexpr int SB = FMT == W_INT4_SYM ? 2 : 4;   // bytes per scale
    // Ring slot u of all waves is an LDS array of its own: the compiler's wait before an
    // LDS read then covers only the copies into the slot read (the array's latest
    // copies), not every copy in flight. After the K loop the waves' partial sums go to
    // slot 0, or to an array of their own when larger.
    static_assert(D <= 8, "one LDS array per ring slot");
    constexpr int SLOTB = NW * XG::SLOT, REDX = red_extra<KS, MT, NT, HX>();
    __shared__ __attribute__((aligned(16))) char xs0[SLOTB];
    __shared__ __attribute__((aligned(16))) char xs1[D > 1 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs2[D > 2 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs3[D > 3 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs4[D > 4 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs5[D > 5 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs6[D > 6 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char xs7[D > 7 ? SLOTB : 16];
    __shared__ __attribute__((aligned(16))) char redx[REDX ? REDX : 16];
    __shared__ uint32_t sl[SCALES == 1 ? sl_words(FMT, MT, NT) : 1];
    char* const xslot[8] = {xs0, xs1, xs2, xs3, xs4, xs5, xs6, xs7};
    f32x4* red = reinterpret_cast<f32x4*>(REDX ? redx : xs0);

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
    // A step reads one group of 16 consecutive columns, words a column's length apart: with
    // 64 fp32 scales per column, all on one bank. When a column is a power-of-two number of
    // words, word i of column c is stored at position i ^ (c & mask) of the column (mask =
    // min(words, 32) - 1), which puts the 16 reads on 16 banks. A copy writes lane l's word
    // to slot l, but each lane may fetch any word, so the permutation costs the copies
    // nothing: lane l fetches the word that belongs in its slot (the swizzle is its own
    // inverse), from the same cache lines.
    const int sbytes = ncols * ngroups * SB, zbytes = ZP ? ncols * ngroups : 0;
    const int swords = (sbytes + 3) >> 2, zwords = (zbytes + 3) >> 2;
    auto col_swizzle = [](int col_bytes, int& shift) {
        const int w = col_bytes >> 2;   // words per column
        shift = __builtin_ctz(w | 0x40000000);
        return col_bytes % 4 == 0 && (w & (w - 1)) == 0 ? (w < 32 ? w : 32) - 1 : 0;
    };
    int s_shift, z_shift;
    const int smask = col_swizzle(ngroups * SB, s_shift);
    const int zmask = ZP ? col_swizzle(ngroups, z_shift) : 0;
    if constexpr (SCALES == 1) {
        // Words past the block's last are copies of its last word (never read); the last
        // word may hold up to 3 bytes past the array's end, inside the same aligned word.
        const uint8_t* sg = reinterpret_cast<const uint8_t*>(scale) + (int64_t)col0 * ngroups * SB;
        for (int q0 = wave * 64; q0 < swords; q0 += 64 * NW) {
            const int w = min(q0 + lane, swords - 1);
            lds_copy4(sg + 4 * (w ^ ((w >> s_shift) & smask)), sl + q0);
        }
        if constexpr (ZP) {
            const uint8_t* zg = zp + (int64_t)col0 * ngroups;
            const int zw0 = (swords + 63) & ~63;
            for (int q0 = wave * 64; q0 < zwords; q0 += 64 * NW) {
                const int w = min(q0 + lane, zwords - 1);
                lds_copy4(zg + 4 * (w ^ ((w >> z_shift) & zmask)), sl + zw0 + q0);
            }
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
    //
    // Weights are loaded with the lanes of a quad on one column (lane l: column
    // 16 j + (l >> 2), chunk l & 3), so that each quad reads one contiguous 4 WB-byte piece:
    // the L1 serves a quad in one request, against one request per lane when the four lanes
    // of a quad sit on four columns as in the MFMA layout (3x the load rate per CU). A lane
    // permute then moves chunk lg of column ln to MFMA lane (ln, lg).
    int woff[NT], soff[NT], sxe[NT], zxe[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int cq = 16 * j + (lane >> 2);
        woff[j] = cq < ncols ? cq * wrow + s0 * G::WSTEP + (lane & 3) * G::WB : OOB;
        const int c = min(16 * j + ln, ncols - 1);   // clamped column
        soff[j] = c * ngroups;                       // its scale and zero index
        sxe[j] = (c & smask) << (SB == 2 ? 1 : 0);   // staged-scale swizzle, in elements
        zxe[j] = (c & zmask) << 2;                   // staged zero-point swizzle, in bytes
    }
    const int wperm = (4 * ln + lg) * 4;   // ds_bpermute byte address of the source lane
    // Activation copies: lane l of copy q takes row q RPC + l / CPR and chunk (l % CPR) ^
    // (row & XM); the row sits in the vector offset, so rows past M read zeros. The
    // swizzle repeats every QV copies.
    int xcv[XG::QV];
#pragma unroll
    for (int v = 0; v < XG::QV; ++v) {
        const int r = v * XG::RPC + lane / XG::CPR;
        xcv[v] = r * K * 2 + s0 * KS * 2 + (((lane % XG::CPR) ^ (r & XG::XM)) * 16);
    }
    // Fragment reads: row 16 i + ln, chunk HN lg + h, in this wave's ring.
    int xfo[HN];
    {
        // with an 8-row ring (HX), lanes of rows 8..15 read rows 0..7 again: those output rows
        // are past M and never stored, and an MFMA output row depends on its own input row only
        const int rr = HX ? (ln & 7) : ln;
        const int row = (rr / XG::RPC) * XG::CSTRIDE + (rr % XG::RPC) * XG::RB;
#pragma unroll
        for (int h = 0; h < HN; ++h)
            xfo[h] = wave * XG::SLOT + row + (((HN * lg + h) ^ (ln & XG::XM)) * 16);
    }

    WR w[D][NT];
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
        char* xs = xslot[u] + wave * XG::SLOT;
#pragma unroll
        for (int q = 0; q < XG::NXC; ++q)
            lds_copy16(xr, (xcv[q % XG::QV] + (q / XG::QV) * XG::QROWS * K * 2) | oob, t * KS * 2,
                       xs + q * XG::CSTRIDE);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int vo = woff[j] | oob;
            if constexpr (G::WB == 8)
                w[u][j] = __builtin_bit_cast(WR, __builtin_amdgcn_raw_buffer_load_b64(wr, vo, t * G::WSTEP, 0));
            else
                w[u][j] = __builtin_bit_cast(WR, __builtin_amdgcn_raw_buffer_load_b128(wr, vo, t * G::WSTEP, 0));
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
                sc[u][j] = (float)reinterpret_cast<const _Float16*>(sl)[e ^ sxe[j]];
            else
                sc[u][j] = reinterpret_cast<const float*>(sl)[e ^ sxe[j]];
            if constexpr (ZP)
                zq[u][j] = reinterpret_cast<const uint8_t*>(sl + zw0)[e ^ zxe[j]];
        }
    };

    f32x4 acc[MT][NT];
    // With group scales and one block of 16 rows (one wave per SIMD, nothing else to run while
    // a step's products finish), a step's scaled add is deferred to the next step: its products
    // (pp) and scale (sp) wait in registers, so the add does not wait for the step's last MFMA
    // (block-asymmetric at 8 rows 6.97 -> 6.52 us; with more row blocks, two waves per SIMD
    // already hide the wait and the extra registers made it slower).
    constexpr bool DEFER = GROUPED && MT == 1;
    f32x4 pp[MT][NT];
    float sp[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[i][j] = f32x4{0, 0, 0, 0};
            pp[i][j] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
    for (int j = 0; j < NT; ++j)
        sp[j] = 0.0f;

    // Vector-memory operations of one step, in issue order: the activation copies, the
    // weight loads, the scale (and zero-point) loads.
    constexpr int NSC = SCALES == 2 ? NT * (ZP ? 2 : 1) : 0;
    constexpr int NL = XG::NXC + NT + NSC;
    // Step u of the ring, with `after` later steps already issued: its activation copies are
    // complete once no more than the step's own later loads and those steps are pending.
    auto compute = [&](int u, auto after) {
        constexpr int pending = NT + NSC + decltype(after)::value * NL;
        __builtin_amdgcn_s_waitcnt(vmcnt_le(pending < 63 ? pending : 63));
        __builtin_amdgcn_sched_barrier(0);
        // the next step's scales are read from LDS one step ahead, so that their latency
        // hides behind this step's work (with a single slot, after this step's products)
        if constexpr (SCALES == 1 && D > 1)
            lds_scales((u + 1) % D);
        f16x8 xa[MT][HN];
        const char* xs = xslot[u];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int h = 0; h < HN; ++h) {
                const f16x8 v = *reinterpret_cast<const f16x8*>(xs + xfo[h] + i * XG::ISTRIDE);
                xa[i][h] = FMT == W_INT4_SYM ? interleave4(v) : v;
            }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            WR wv;
#pragma unroll
            for (int d = 0; d < G::WB / 4; ++d)
                wv[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(wperm, (int)w[u][j][d]);
            f16x8 wb[HN];
            if constexpr (FMT == W_INT4_SYM) {
#pragma unroll
                for (int h = 0; h < HN; ++h)
                    wb[h] = int4_to_f16(wv[h]);
            } else if constexpr (FMT == W_INT8_SYM) {
                bytes_to_f16(wv, 0x80808080u, (_Float16)1152.0f, wb[0], wb[1]);
            } else {
                const _Float16 z = (_Float16)(float)(1024 + zq[u][j]);
                if constexpr (NT == 4)
                    bytes_to_f16_pairs(wv, 0u, f16x2{z, z}, wb[0], wb[1]);
                else
                    bytes_to_f16(wv, 0u, z, wb[0], wb[1]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if constexpr (GROUPED) {
                    f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][0], wb[0], f32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int h = 1; h < HN; ++h)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][h], wb[h], p, 0, 0, 0);
                    if constexpr (DEFER) {
                        acc[i][j] += sp[j] * pp[i][j];
                        pp[i][j] = p;
                        if (i == MT - 1)
                            sp[j] = sc[u][j];
                    } else {
                        acc[i][j] += sc[u][j] * p;
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < HN; ++h)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i][h], wb[h], acc[i][j], 0, 0, 0);
                }
            }
        }
        if constexpr (SCALES == 1 && D == 1)
            lds_scales(0);
    };

#pragma unroll
    for (int u = 0; u < D; ++u)
        load(u, u);
    if constexpr (SCALES == 1) {
        // This wave's copies into LDS are older than the D steps of loads just issued; then
        // the barrier makes every wave's copies visible.
        constexpr int younger = D * NL;
        __builtin_amdgcn_s_waitcnt(vmcnt_le(younger < 63 ? younger : 63));
        asm volatile("s_barrier" ::: "memory");
        lds_scales(0);
    }
    // sched_barrier keeps each step's work together, so that the registers of one step's
    // products are free before the next step starts.
    for (int tb = 0; tb + D < TP; tb += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            compute(u, std::integral_constant<int, D - 1>{});
            // the slot's reads have completed: their values feed this step's MFMAs
            __builtin_amdgcn_sched_barrier(0);
            load(u, tb + D + u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    static_for<D>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        compute(u, std::integral_constant<int, D - 1 - u>{});
        __builtin_amdgcn_sched_barrier(0);
    });

    if constexpr (DEFER) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[i][j] += sp[j] * pp[i][j];
    }
    // The waves' partial sums meet in LDS (over the rings: every wave must be done with
    // its ring first); wave w then finishes blocks b = w (mod NW). Their per-column
    // factors are loaded first, before any store: a vector-memory wait also waits for the
    // stores already issued, so a load between two blocks' stores would hold the second
    // block until the first one's stores had completed.
    constexpr int NB = (MT * NT + NW - 1) / NW;   // blocks per wave, at most
    float cscale[NB], cbias[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int b = wave + k * NW;
        const int n = col0 + min(16 * (b % NT) + ln, ncols - 1);
        cscale[k] = 1.0f;
        cbias[k] = 0.0f;
        if (b < MT * NT) {
            if constexpr (!GROUPED)
                cscale[k] = reinterpret_cast<const float*>(scale)[n];
            if (bias)
                cbias[k] = bias[n];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            red[((wave * MT + i) * NT + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    // The factors have arrived (nothing else is pending): said once here, so that the
    // compiler sees no load outstanding at the per-row store branches below.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    // Output element r of block (i, j) in lane l is C[4 (l >> 4) + r][l & 15]. The
    // activation is uniform: one store loop per kind.
    auto finish = [&](auto act_c) {
        constexpr int ACT = decltype(act_c)::value;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int b = wave + k * NW;
            if (b >= MT * NT)
                break;
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
                v *= cscale[k];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * i + 4 * lg + r;
                if (m < M)
                    Y[(int64_t)m * N + n] = (_Float16)activation<ACT, true>(v[r] + cbias[k]);
            }
        }
    };
    if (act == ACT_GELU)
        finish(std::integral_constant<int, ACT_GELU>{});
    else if (act == ACT_SILU)
        finish(std::integral_constant<int, ACT_SILU>{});
    else
        finish(std::integral_constant<int, ACT_NONE>{});
}

template <int FMT, int KS, int MT, int NT, int SCALES, bool HX>
ql_status launch_cfg(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                     int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                     int cols, int act, hipStream_t stream) {
    constexpr int D = ring_depth<FMT, KS, MT, NT, SCALES, HX>();
    const dim3 grid((unsigned)((N + cols - 1) / cols)), block(64 * nwaves<MT>());
    hipLaunchKernelGGL((wonly_kernel<FMT, KS, MT, NT, SCALES, D, HX>), grid, block, 0, stream,
                       reinterpret_cast<const _Float16*>(x), reinterpret_cast<const uint8_t*>(codes),
                       scale, zp, (int)group, bias, reinterpret_cast<_Float16*>(y), (int)M, (int)N,
                       (int)K, cols, act);
    return launch_status();
}

template <int FMT, int KS, int MT, int SCALES, bool HX>
ql_status launch_nt(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                    int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                    int cols, int act, hipStream_t stream) {
    if (cols <= 16)
        return launch_cfg<FMT, KS, MT, 1, SCALES, HX>(x, codes, scale, zp, group, bias, y, M, N, K, cols, act, stream);
    if (cols <= 32)
        return launch_cfg<FMT, KS, MT, 2, SCALES, HX>(x, codes, scale, zp, group, bias, y, M, N, K, cols, act, stream);
    return launch_cfg<FMT, KS, MT, 4, SCALES, HX>(x, codes, scale, zp, group, bias, y, M, N, K, cols, act, stream);
}

template <int FMT, int KS, int MT, bool HX = false>
ql_status launch_mt(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                    int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                    bool grouped, int act, hipStream_t stream) {
    // Columns per workgroup: an equal share per CU, in multiples of 8, at most 64.
    int64_t cols = (N + cu_count() - 1) / cu_count();
    cols = (cols + 7) / 8 * 8;
    if (cols > 64)
        cols = 64;
    if (!grouped)
        return launch_nt<FMT, KS, MT, 0, HX>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, act, stream);
    // The scale block (and zero-point block after it, at a 64-word boundary) must fit in LDS.
    const int64_t ng = K / group, sb = FMT == W_INT4_SYM ? 2 : 4;
    const int64_t words = ((cols * ng * sb + 3) / 4 + 63) / 64 * 64 + (FMT == W_UINT8_ZP ? (cols * ng + 3) / 4 : 0);
    const int nt = cols <= 16 ? 1 : cols <= 32 ? 2 : 4;   // as launch_nt picks it
    if (words + 63 <= sl_words(FMT, MT, nt))
        return launch_nt<FMT, KS, MT, 1, HX>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, act, stream);
    return launch_nt<FMT, KS, MT, 2, HX>(x, codes, scale, zp, group, bias, y, M, N, K, (int)cols, act, stream);
}

template <int FMT, int KS>
ql_status launch_rows(const void* x, const void* codes, const void* scale, const uint8_t* zp,
                      int64_t group, const float* bias, void* y, int64_t M, int64_t N, int64_t K,
                      bool grouped, int act, hipStream_t stream) {
    // Rows are processed 64 at a time (MT = 4 blocks of 16); smaller M uses fewer blocks (33..48
    // rows on three blocks rather than four: 4-16% faster, e.g. int4 at 48 rows, N = 14336,
    // 19.4 -> 16.9 us).
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
        const int64_t mc = M - m0 < 64 ? M - m0 : 64;
        const void* xs = reinterpret_cast<const _Float16*>(x) + m0 * K;
        void* ys = reinterpret_cast<_Float16*>(y) + m0 * N;
        ql_status st;
        if (mc <= 8)
            st = launch_mt<FMT, KS, 1, true>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, act, stream);
        else if (mc <= 16)
            st = launch_mt<FMT, KS, 1>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, act, stream);
        else if (mc <= 32)
            st = launch_mt<FMT, KS, 2>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, act, stream);
        else if (mc <= 48)
            st = launch_mt<FMT, KS, 3>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, act, stream);
        else
            st = launch_mt<FMT, KS, 4>(xs, codes, scale, zp, group, bias, ys, mc, N, K, grouped, act, stream);
        if (st != QL_OK)
            return st;
    }
    return QL_OK;
}

}  // namespace

ql_status launch_wonly(const void* x, const void* codes, int fmt, const void* scale,
                       const uint8_t* zp, int64_t group, const float* bias, void* y, int64_t M,
                       int64_t N, int64_t K, int act, hipStream_t stream) {
    if (M == 0 || N == 0)
        return QL_OK;
    switch (fmt) {
    case W_INT8_SYM:
        if (group == 0 || group == K)
            return launch_rows<W_INT8_SYM, 64>(x, codes, scale, zp, K, bias, y, M, N, K, false, act, stream);
        return launch_rows<W_INT8_SYM, 64>(x, codes, scale, zp, group, bias, y, M, N, K, true, act, stream);
    case W_UINT8_ZP:
        return launch_rows<W_UINT8_ZP, 64>(x, codes, scale, zp, group == 0 ? K : group, bias, y, M, N,
                                           K, true, act, stream);
    default:
        // 128-k steps (16-byte loads) when a step never straddles a group
        if (group % 128 == 0 && K % 128 == 0)
            return launch_rows<W_INT4_SYM, 128>(x, codes, scale, zp, group, bias, y, M, N, K, true, act, stream);
        return launch_rows<W_INT4_SYM, 64>(x, codes, scale, zp, group, bias, y, M, N, K, true, act, stream);
    }
}

}  // namespace ql
