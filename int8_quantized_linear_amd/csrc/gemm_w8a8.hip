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
// Tiles are 256 x 256 per workgroup of 4 waves (2 x 2); each wave owns a 128 x 128 block
// of accumulators = 4 x 4 v_mfma_i32_32x32x32_i8 blocks (256 accumulator registers per
// lane). K advances 64 bytes per step through a ring of LDS stages that global -> LDS
// direct copies (no register staging) fill ahead of use; each step reads the next
// step's MFMA fragments while its own MFMAs run, with one barrier per step. The tile
// size is set by L2 -> CU bandwidth: a tile moves (BM + BN) bytes per k for BM * BN
// multiply-adds. When the last round of 256 x 256 tiles would leave CUs idle, its N
// panels are cut into 128 x 256 tiles instead.
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BK = 64;
constexpr int NTHR = 256;   // threads of the 64-byte ring path
#ifndef GEMM_WAVES_K128
#define GEMM_WAVES_K128 8
#endif
#ifndef GEMM_PINGPONG
#define GEMM_PINGPONG 1
#endif

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt immediate that waits until at most n vector-memory operations are pending
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// Workgroup barrier without a memory fence: __syncthreads() would also wait for every
// pending global -> LDS copy, including the stages still being prefetched. Each wave
// instead waits (vmcnt) for its own copies of the stage about to be read, and LDS reads
// are complete before the MFMAs that consume them, so after the barrier the stage is
// visible and the oldest buffer is free. The "memory" clobber keeps the compiler from
// moving LDS accesses across the barrier.
__device__ inline void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane
// l's bytes land at l * 16 past the wave-uniform LDS address. Compiled in the device pass
// only: in the host pass the builtin makes clang drop the kernel's launch stub silently.
__device__ inline void lds_copy16(const void* g, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
#endif
}

// Row r of a staged tile is 64 bytes = four 16-byte chunks. Chunk c of row r is stored
// at chunk position c ^ rowhash(r), so that the 16 rows read together by one fragment
// load fall in distinct bank groups (for 8- and for 16-lane LDS access phases).
__device__ inline int rowhash(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ inline int swz(int r, int c) { return r * BK + ((c ^ rowhash(r)) << 4); }

// 4 bytes per lane from global memory straight into LDS (global_load_lds_dword): lane l's
// word lands at l * 4 past the wave-uniform LDS address.
__device__ inline void lds_copy4(const void* g, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 4, 0, 0);
#endif
}

// Bytes of the K ring at the start of the LDS allocation (three stages of a 128 x 256 tile
// with 128-byte k-steps); the tile's scales follow it: x_scale of its 256 rows, then
// w_scale and bias of its 256 columns (fp32 each).
constexpr int RING_BYTES = 3 * 384 * 128;
constexpr int SCALE_BYTES = 3 * 256 * 4;

// Waves 0-3 each copy 64 of the tile's x_scale, w_scale and bias entries into LDS
// (indices clamped into range; entries past M or N are never used). Issued before the K
// loop's first copies, so every wait of the loop also covers them; the epilogue's barrier
// makes them visible to all waves. Without a bias, w_scale is copied in its place (unused).
__device__ inline void issue_scales(const float* xs, const float* ws, const float* bias, int M,
                                    int N, int m0, int n0, int wave, int lane, int8_t* smem) {
    if (wave >= 4)
        return;
    int8_t* sc = smem + RING_BYTES + wave * 256;
    const int i = wave * 64 + lane;
    lds_copy4(xs + min(m0 + i, M - 1), sc);
    lds_copy4(ws + min(n0 + i, N - 1), sc + 1024);
    lds_copy4((bias != nullptr ? bias : ws) + min(n0 + i, N - 1), sc + 2048);
}

// Epilogue: the accumulators are dequantized (y = acc * x_scale[m] * w_scale[n] + bias[n])
// in registers and leave through LDS, one 32-row band of the wave's block at a time, so
// that global stores are whole 16-byte pieces of contiguous row segments rather than
// 2- or 4-byte scattered writes. Element e of block (i, j) in lane l is
// C[8 (e >> 2) + 4 (l >> 5) + (e & 3)][l & 31] of that 32 x 32 block.
// Stores go through a buffer descriptor whose size ends at row M: the hardware drops
// stores of rows past M, and a column piece past N gets an offset beyond the size, so no
// store needs a branch.
template <int WM, int WN, int FM, int FN, int YMODE, int NWV>
__device__ __forceinline__ void store_tile(const i32x16 (&acc)[FM][FN], bool has_bias,
                                           void* __restrict__ Y, int M, int N, int mrow0,
                                           int ncol0, int lm0, int ln0, int wave, int lane,
                                           int8_t* smem) {
    using OutT = typename std::conditional<YMODE == Y_F16, _Float16,
                 typename std::conditional<YMODE == Y_F32, float, int32_t>::type>::type;
    constexpr int SZ = sizeof(OutT);
    constexpr int VEC = 16 / SZ;                    // elements per 16-byte store
    constexpr int ROWB = WN * SZ + 32;              // staged row, padded: rows r, r + 4 differ in bank half
    constexpr int LPR = WN * SZ / 16;               // lanes per staged row
    constexpr int RPI = 64 / LPR;                   // rows per read / store instruction
    constexpr int NRD = 32 / RPI;                   // reads (and stores) per band
    static_assert(NWV * 32 * ROWB <= RING_BYTES, "output staging fits the LDS ring");
    // Descriptor sizes are capped at LIM = 2^30 bytes, which no in-range offset reaches
    // (32 rows of at most 2^23 4-byte values); a column piece past N is sent to offset
    // row + LIM, at or past the size, and row + LIM stays below 2^31.
    constexpr int LIM = 1 << 30;

    barrier_no_fence();   // the ring is no longer read; every wave's scale copies landed
    int8_t* stage = smem + wave * 32 * ROWB;
    const float* sx = reinterpret_cast<const float*>(smem + RING_BYTES);
    const float* sw = sx + 256;
    const float* sb = sx + 512;
    float wsv[FN], bv[FN];
    if constexpr (YMODE != Y_I32) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c = ln0 + 32 * j + (lane & 31);
            wsv[j] = sw[c];
            bv[j] = has_bias ? sb[c] : 0.0f;
        }
    }
    const bool vec_ok = (N % VEC) == 0;   // rows start 16-byte aligned
    // byte offset of this lane's 16-byte piece in the first row it stores of a band
    const int ncol = ncol0 + (lane % LPR) * VEC;
    const int lane_off = (lane / LPR) * N * SZ + (ncol < N ? ncol * SZ : LIM);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        float xsv[16];
        if constexpr (YMODE != Y_I32) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(sx + lm0 + 32 * i + 8 * g + 4 * (lane >> 5));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xsv[4 * g + q] = v[q];
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                OutT v;
                if constexpr (YMODE == Y_I32)
                    v = acc[i][j][e];
                else
                    v = (OutT)((float)acc[i][j][e] * xsv[e] * wsv[j] + bv[j]);
                *reinterpret_cast<OutT*>(stage + r * ROWB + (32 * j + (lane & 31)) * SZ) = v;
            }
        }
        // The wave's LDS operations complete in order, so its reads below see all of its
        // writes above; this only keeps the compiler from reordering them.
        asm volatile("" ::: "memory");
        u32x4 rv[NRD];
#pragma unroll
        for (int p = 0; p < NRD; ++p) {
            const int r = p * RPI + lane / LPR, c = (lane % LPR) * VEC;
            rv[p] = *reinterpret_cast<const u32x4*>(stage + r * ROWB + c * SZ);
        }
        const int row0 = mrow0 + 32 * i;
        const int64_t left = (int64_t)(M - row0) * N * SZ;   // bytes from row0 to the end
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<int8_t*>(Y) + (int64_t)row0 * N * SZ, 0,
            (int)(left <= 0 ? 0 : (left < LIM ? left : LIM)), 0x00020000);
        if (vec_ok) {
#pragma unroll
            for (int p = 0; p < NRD; ++p)
                __builtin_amdgcn_raw_buffer_store_b128(rv[p], rs, lane_off + p * RPI * N * SZ, 0, 0);
        } else {
            const int n = ncol0 + (lane % LPR) * VEC;
#pragma unroll
            for (int p = 0; p < NRD; ++p) {
                const int roff = (p * RPI + lane / LPR) * N * SZ;
                const OutT* pv = reinterpret_cast<const OutT*>(&rv[p]);
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    const int off = roff + (n + q < N ? (n + q) * SZ : LIM);
                    if constexpr (SZ == 2)
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, pv[q]), rs, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pv[q]), rs, off, 0, 0);
                }
            }
        }
        asm volatile("" ::: "memory");   // the next band's writes follow these reads
    }
}

// One output tile of BM x BN (BM = 256 or 128, BN = 256) computed by the workgroup's 4
// waves laid out 2 x 2; each wave owns (BM/2) x (BN/2) = FM x FN blocks of 32 x 32
// accumulators (v_mfma_i32_32x32x32_i8, 16 int32 per lane each). K advances BK = 64
// bytes per step through a ring of STAGES LDS buffers (two 32-deep k-substeps per step).
template <int BM, int BN, int STAGES, int YMODE>
__device__ __forceinline__ void gemm_tile(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                          const int8_t* __restrict__ B, const float* __restrict__ ws,
                                          const float* __restrict__ bias, void* __restrict__ Y, int M,
                                          int N, int K, int m0, int n0, int8_t* smem) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int STAGE_A = BM * BK, STAGE = (BM + BN) * BK;
    constexpr int LA = BM * BK / 16 / NTHR, LB = BN * BK / 16 / NTHR;  // copies per thread
    constexpr int LOADS = LA + LB;
    static_assert(STAGES >= 3, "the ring needs a buffer being read, one landing, one free");
    static_assert(STAGES * STAGE <= RING_BYTES, "the ring fits its LDS");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int KT = K / BK;

    // Global -> LDS copy. Wave w fills a contiguous run of 16-byte slots of each operand's
    // stage, 64 slots per instruction; lane l of an instruction lands in slot base + l.
    // Slot s holds row s >> 2 at chunk position s & 3, i.e. logical chunk
    // (s & 3) ^ rowhash(row). Rows past M or N are clamped to the last row (their results
    // are never stored).
    const int8_t* ga[LA];
    const int8_t* gb[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int slot = wave * (LA * 64) + i * 64 + lane;
        const int r = slot >> 2, c = (slot & 3) ^ rowhash(slot >> 2);
        ga[i] = A + (int64_t)min(m0 + r, M - 1) * K + c * 16;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int slot = wave * (LB * 64) + i * 64 + lane;
        const int r = slot >> 2, c = (slot & 3) ^ rowhash(slot >> 2);
        gb[i] = B + (int64_t)min(n0 + r, N - 1) * K + c * 16;
    }
    // Copies stage kt (its K columns clamped to the last stage) into ring buffer kt % STAGES.
    auto issue = [&](int kt) {
        int8_t* st = smem + (kt % STAGES) * STAGE;
        const int k0 = min(kt, KT - 1) * BK;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            lds_copy16(ga[i] + k0, st + (wave * LA + i) * 1024);
#pragma unroll
        for (int i = 0; i < LB; ++i)
            lds_copy16(gb[i] + k0, st + STAGE_A + (wave * LB + i) * 1024);
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // Fragment reads: for k-substep ks, lane l takes row (l & 31) of a 32-row block and
    // logical chunk 2 ks + (l >> 5) of the 64-byte step; A and B use the same
    // k <-> (lane, byte) assignment, so their products pair the same k. rowhash depends on
    // the low 4 row bits only, so a wave's blocks are one base address plus multiples of 2 KB.
    const int fa_off = wm * WM * BK, fb_off = STAGE_A + wn * WN * BK;
    const int fr = lane & 31;
    const int f_off0 = swz(fr, lane >> 5), f_off1 = swz(fr, 2 + (lane >> 5));
    typedef i32x4 Frag[2][FM + FN];   // [ks][A blocks then B blocks]
    auto read_frags = [&](int kt, Frag& f) {
        const int8_t* st = smem + (kt % STAGES) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int fo = ks ? f_off1 : f_off0;
            // B first: the next step's first MFMAs use A block 0 with every B block
#pragma unroll
            for (int j = 0; j < FN; ++j)
                f[ks][FM + j] = *reinterpret_cast<const i32x4*>(st + fb_off + fo + j * 32 * BK);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                f[ks][i] = *reinterpret_cast<const i32x4*>(st + fa_off + fo + i * 32 * BK);
        }
    };
    auto mfmas = [&](const Frag& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[ks][i], f[ks][FM + j], acc[i][j], 0, 0, 0);
    };

    // Step kt: wait until stage kt+1 has landed (only the copies of the stages after it
    // may still be pending), barrier, issue stage kt+STAGES-1 into the buffer that held
    // stage kt-1 (every wave consumed those fragments before the barrier), read stage
    // kt+1's fragments, and run stage kt's MFMAs with the copies and reads spread among
    // them. Past the last stage the copies repeat the last stage (the buffers they fill
    // are never read), so every step has the same shape. sched_barrier(0) keeps steps
    // from being interleaved with each other. Before step kt's wait, stages
    // 0 .. kt+STAGES-2 have been issued.
    constexpr int NMF = 2 * FM * FN, NDS = 2 * (FM + FN);
    auto step = [&](int kt, const Frag& cur, Frag& nxt) {
        __builtin_amdgcn_s_waitcnt(vmcnt_le((STAGES - 3) * LOADS));
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + STAGES - 1);
        read_frags(kt + 1, nxt);
        mfmas(cur);
#pragma unroll
        for (int g = 0; g < LOADS; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                  // VMEM (copy)
            __builtin_amdgcn_sched_group_barrier(0x100, NDS / LOADS, 0);        // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, NMF / LOADS, 0);        // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NDS % LOADS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF % LOADS, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Steps run in pairs over two fragment register sets. With an odd number of steps a
    // virtual step -1 of zero fragments comes first. Before the first step k0 the copies
    // of stages k0+1 .. k0+STAGES-2 are the ones pending.
    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, M, N, m0, n0, wave, lane, smem);
    Frag f0, f1;
    int k0;
    if (KT & 1) {
        k0 = -1;
#pragma unroll
        for (int s = 0; s < STAGES - 2; ++s)
            issue(s);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < FM + FN; ++i)
                f0[ks][i] = i32x4{0, 0, 0, 0};
    } else {
        k0 = 0;
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            issue(s);
        __builtin_amdgcn_s_waitcnt(vmcnt_le((STAGES - 2) * LOADS));
        barrier_no_fence();
        read_frags(0, f0);
    }
    for (int kt = k0; kt < KT; kt += 2) {
        step(kt, f0, f1);
        step(kt + 1, f1, f0);   // reads past the end on the last pair: never used
    }
    // No copy into LDS may still be in flight when the workgroup's LDS is released.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));

    store_tile<WM, WN, FM, FN, YMODE, 4>(acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN, wm * WM,
                                         wn * WN, wave, lane, smem);
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

// The same tile with 128-byte k-steps (for K % 128 == 0): each copied row piece is a whole
// 128-byte line, which the L2 -> CU path delivers at about twice the rate of half lines.
// Two LDS stages of (BM + BN) x 128 bytes. The workgroup's WGM x WGN waves each own a
// (BM / WGM) x (BN / WGN) block; with 8 waves (two per SIMD) a wave's block is half as
// wide, which costs half again as many LDS fragment reads per multiply, but two waves per
// SIMD issue LDS reads about twice as fast as one and cover each other's waits.
// Fragments are read two 32-deep substeps ahead of the MFMAs that use them (four
// fragment register sets), so an LDS read has two substeps to return. Halfway through
// stage kt every fragment of stage kt has been read: each wave waits for its own LDS
// reads and for its copies of stage kt + 1, and after a barrier stage kt's buffer takes
// the copies of stage kt + 2 while the reads move on to stage kt + 1.
template <int BM, int BN, int WGM, int WGN, int YMODE>
__device__ __forceinline__ void gemm_tile128(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                             const int8_t* __restrict__ B, const float* __restrict__ ws,
                                             const float* __restrict__ bias, void* __restrict__ Y,
                                             int M, int N, int K, int m0, int n0, int8_t* smem) {
    constexpr int BKL = 128;
    constexpr int NWV = WGM * WGN, NT = 64 * NWV;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int STAGE_A = BM * BKL, STAGE = (BM + BN) * BKL;
    constexpr int LA = BM * BKL / 16 / NT, LB = BN * BKL / 16 / NT;  // copies per thread
    constexpr int LOADS = LA + LB;
    static_assert(LA * 16 * NT == BM * BKL && LB * 16 * NT == BN * BKL, "copies divide evenly");
    static_assert(2 * STAGE <= RING_BYTES, "two stages fit the LDS allocation");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int KT = K / BKL;

    // Copy slots: slot s holds row s >> 3 at chunk position s & 7, i.e. logical chunk
    // (s & 7) ^ h128(row); lane l of an instruction lands in slot base + l. Rows past M or
    // N are clamped to the last row (their results are never stored). The descriptors
    // start at the tile's first row, so offsets stay below 256 K bytes.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A) + (int64_t)m0 * K, 0, (int)((int64_t)(M - m0 < BM ? M - m0 : BM) * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B) + (int64_t)n0 * K, 0, (int)((int64_t)(N - n0 < BN ? N - n0 : BN) * K), 0x00020000);
    int va[LA], vb[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int slot = wave * (LA * 64) + i * 64 + lane;
        const int r = slot >> 3, c = (slot & 7) ^ h128(slot >> 3);
        va[i] = min(r, M - 1 - m0) * K + c * 16;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int slot = wave * (LB * 64) + i * 64 + lane;
        const int r = slot >> 3, c = (slot & 7) ^ h128(slot >> 3);
        vb[i] = min(r, N - 1 - n0) * K + c * 16;
    }
    // Copies q0 .. q1 - 1 (A's then B's) of stage kt (clamped to the last stage) into
    // buffer kt & 1.
    auto issue_part = [&](int kt, int q0, int q1) {
        int8_t* st = smem + (kt & 1) * STAGE;
        const int k0 = __builtin_amdgcn_readfirstlane(min(kt, KT - 1) * BKL);
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            if (q < LA)
                lds_copy16_buf(ra, va[q], k0, st + (wave * LA + q) * 1024);
            else
                lds_copy16_buf(rb, vb[q - LA], k0, st + STAGE_A + (wave * LB + q - LA) * 1024);
        }
    };
    auto issue = [&](int kt) { issue_part(kt, 0, LOADS); };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // Fragment of substep u (stage u >> 2, k-substep u & 3): lane l takes row (l & 31) of a
    // 32-row block and logical chunk 2 (u & 3) + (l >> 5); A and B use the same
    // k <-> (lane, byte) assignment. h128 depends on the low 4 row bits only.
    const int lr = lane & 31;
    const int fa_base = wm * WM * BKL + lr * BKL, fb_base = STAGE_A + wn * WN * BKL + lr * BKL;
    typedef i32x4 Frag[FM + FN];   // A blocks then B blocks
    auto read = [&](int u, Frag& f) {
        const int8_t* st = smem + ((u >> 2) & 1) * STAGE;
        const int co = ((2 * (u & 3) + (lane >> 5)) ^ h128(lr)) << 4;
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f[FM + j] = *reinterpret_cast<const i32x4*>(st + fb_base + co + j * 32 * BKL);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f[i] = *reinterpret_cast<const i32x4*>(st + fa_base + co + i * 32 * BKL);
    };
    auto mfma = [&](const Frag& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[i], f[FM + j], acc[i][j], 0, 0, 0);
    };
    constexpr int NMF = FM * FN, NDS = FM + FN;
    constexpr int CPS = (LOADS + 3) / 4;   // copies per substep when a stage's are spread over 4
    // A substep: the MFMAs of substep u with the reads of substep u + 2 and copies
    // q0 .. q1 - 1 of stage kc spread among them, so that neither the LDS queue nor the
    // copy path takes a burst that would hold up the wave's MFMA issue.
    auto sub = [&](int u, const Frag& cur, Frag& ahead, int kc, int q0, int q1) {
        read(u + 2, ahead);
        issue_part(kc, q0, q1);
        mfma(cur);
        constexpr int G = NDS / 2, Q = NMF / G;
#pragma unroll
        for (int g = 0; g < G - 1; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, Q, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (copy), if any
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - (G - 1) * Q, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, CPS, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NDS - (G - 1) * 2, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, M, N, m0, n0, wave, lane, smem);
    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(LOADS) & ~(0xF << 8));   // stage 0 landed (this wave's copies)
    barrier_no_fence();
    Frag f0, f1, f2, f3;
    read(0, f0);
    read(1, f1);
    sub(0, f0, f2, 0, 0, 0);
    sub(1, f1, f3, 0, 0, 0);
    // Each iteration runs the second half of stage kt and the first half of stage kt + 1.
    // It starts right after a wait and barrier that leave no LDS read pending (so the
    // compiler's waits inside count exactly): stage kt + 1 is complete in LDS and stage
    // kt is fully read, so its buffer takes the copies of stage kt + 2.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0) & ~(0xF << 8));   // vmcnt(0) lgkmcnt(0)
    barrier_no_fence();
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int u = 4 * kt;
        // stage kt + 2's copies, a quarter per substep (past the end they repeat the last
        // stage, never read)
        sub(u + 2, f2, f0, kt + 2, 0, CPS);
        sub(u + 3, f3, f1, kt + 2, CPS, min(2 * CPS, LOADS));
        sub(u + 4, f0, f2, kt + 2, min(2 * CPS, LOADS), min(3 * CPS, LOADS));
        sub(u + 5, f1, f3, kt + 2, min(3 * CPS, LOADS), LOADS);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0) & ~(0xF << 8));
        barrier_no_fence();
    }
    // the last stage's second half
    mfma(f2);
    mfma(f3);
    // No copy into LDS may still be in flight when the LDS is reused or released.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    store_tile<WM, WN, FM, FN, YMODE, NWV>(acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN,
                                           wm * WM, wn * WN, wave, lane, smem);
}

// A BM x BN tile (256 x 256 or 128 x 256) on 8 waves with a ping-pong schedule
// (K % 128 == 0). Waves 0-3
// (group 0) and 4-7 (group 1) put one wave of each group on every SIMD, and the two
// groups alternate between phases separated by workgroup barriers: in each phase one
// group issues nothing but the 32 MFMAs of a whole 128-deep stage (its fragments already
// in registers), while the other group reads the next stage's fragments from LDS and,
// for group 0, issues the copies of the stage after. The MFMA stream of a SIMD then never
// waits behind an LDS or copy instruction of its own wave. Wave w owns the (BM / 2) x
// (BN / 4) block at rows (BM / 2) (w & 1), columns (BN / 4) (w >> 1).
//
// Phase 2j:   group 0 runs stage j's MFMAs, then waits for its copies of stage j + 1;
//             group 1 reads stage j's fragments.
// Phase 2j+1: group 0 issues the copies of stage j + 2 into stage j's buffer (stage j
//             was read in phases 2j - 1 and 2j) and reads stage j + 1's fragments;
//             group 1 runs stage j's MFMAs.
// Copies thus have two phases (one stage of MFMA time) to land.
template <int BM, int BN, int YMODE>
__device__ __forceinline__ void gemm_tile_pp(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                             const int8_t* __restrict__ B, const float* __restrict__ ws,
                                             const float* __restrict__ bias, void* __restrict__ Y,
                                             int M, int N, int K, int m0, int n0, int8_t* smem) {
    constexpr int BKL = 128;
    constexpr int WM = BM / 2, WN = BN / 4, FM = WM / 32, FN = WN / 32;
    constexpr int STAGE_A = BM * BKL, STAGE = (BM + BN) * BKL;
    constexpr int CA = BM / 32, CB = BN / 32;   // copies of A and of B per group-0 wave (8 rows each)
    static_assert(2 * STAGE <= RING_BYTES, "two stages fit the LDS allocation");
    static_assert(FM >= 1 && FN >= 1 && CA % 2 == 0 && CB % 2 == 0, "tile shape");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm = wave & 1, wn = wave >> 1;
    const int KT = K / BKL;

    // Group-0 wave q copies rows (BM / 4) q .. of A and (BN / 4) q .. of B: copy c moves 8
    // rows x 128 bytes, lane l row R q + 8 c + (l >> 3), logical chunk (l & 7) ^ h128(row)
    // (landing at chunk position l & 7). Rows past M or N read as zeros (outside the
    // descriptor).
    const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A) + (int64_t)m0 * K, 0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B) + (int64_t)n0 * K, 0, rows_b * K, 0x00020000);
    // Row R q + 8 c + (l >> 3) (R a multiple of 16) has h128 = ((l >> 3) & 7) ^ (c & 1), so
    // a lane's offset is one of two values plus 8 c rows, which goes with the k-step in the
    // scalar offset. A row past the descriptor's end gets an offset at or past it (also
    // with the scalar part added, which stays below 2^31): the hardware returns zeros.
    const int cra = (BM / 4) * q + (lane >> 3), crb = (BN / 4) * q + (lane >> 3);
    const int cx = (lane & 7) ^ ((lane >> 3) & 7);
    const int va0 = cra * K + (cx << 4), va1 = cra * K + ((cx ^ 1) << 4);
    const int vb0 = crb * K + (cx << 4), vb1 = crb * K + ((cx ^ 1) << 4);
    auto copies = [&](int kt, int buf) {
        int8_t* st = smem + buf * STAGE;
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int so = __builtin_amdgcn_readfirstlane(kt * BKL + 8 * c * K);
            lds_copy16_buf(ra, cra + 8 * c < rows_a ? ((c & 1) ? va1 : va0) : 0x7FFFFFF0, so,
                           st + ((BM / 4) * q + 8 * c) * BKL);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int so = __builtin_amdgcn_readfirstlane(kt * BKL + 8 * c * K);
            lds_copy16_buf(rb, crb + 8 * c < rows_b ? ((c & 1) ? vb1 : vb0) : 0x7FFFFFF0, so,
                           st + STAGE_A + ((BN / 4) * q + 8 * c) * BKL);
        }
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // Fragments of a whole stage: F[ks][A blocks then B blocks], ks the 32-deep substep.
    const int lr = lane & 31;
    const int fa_base = wm * WM * BKL + lr * BKL, fb_base = STAGE_A + wn * WN * BKL + lr * BKL;
    i32x4 F[4][FM + FN];
    auto read_stage = [&](int kt) {
        const int8_t* st = smem + (kt & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int co = ((2 * ks + (lane >> 5)) ^ h128(lr)) << 4;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                F[ks][FM + j] = *reinterpret_cast<const i32x4*>(st + fb_base + co + j * 32 * BKL);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                F[ks][i] = *reinterpret_cast<const i32x4*>(st + fa_base + co + i * 32 * BKL);
        }
    };
    auto mfma_stage = [&]() {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F[ks][i], F[ks][FM + j], acc[i][j], 0, 0, 0);
    };

    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, M, N, m0, n0, wave, lane, smem);
    if (grp == 0) {
        copies(0, 0);
        copies(min(1, KT - 1), 1);   // with one stage, a second copy of it (never read)
        __builtin_amdgcn_s_waitcnt(vmcnt_le(CA + CB) & ~(0xF << 8));   // stage 0 landed
    }
    barrier_no_fence();
    // Each group runs its own straight-line loop; both execute the same barriers in the
    // same order (two per stage). sched_barrier keeps the compiler from moving MFMAs (which
    // the barrier's memory clobber does not pin) from one phase into another.
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
    };
    if (grp == 0) {
        read_stage(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0)
        phase_end();
        for (int j = 0; j < KT; ++j) {
            // phase 2j: stage j's MFMAs, then this wave's copies of stage j + 1 have landed
            mfma_stage();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
            phase_end();
            // phase 2j + 1: copies of stage j + 2 into stage j's buffer, reads of stage j + 1
            // (past the end they repeat the last stage into the free buffer: never used)
            copies(min(j + 2, KT - 1), j & 1);
            read_stage(min(j + 1, KT - 1));
            __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0)
            phase_end();
        }
    } else {
        phase_end();   // while group 0 reads stage 0
        for (int j = 0; j < KT; ++j) {
            // phase 2j: reads of stage j
            read_stage(j);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(0xF << 8));   // lgkmcnt(0)
            phase_end();
            // phase 2j + 1: stage j's MFMAs
            mfma_stage();
            phase_end();
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    store_tile<WM, WN, FM, FN, YMODE, 8>(acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN,
                                         wm * WM, wn * WN, wave, lane, smem);
}

// A 128 x 256 tile on 8 waves with K split between two groups (K % 128 == 0). Group 0
// (waves 0-3) accumulates the even 128-deep stages and group 1 (waves 4-7) the odd ones,
// each over the whole tile with a 2 x 2 arrangement of 64 x 128 wave blocks, so one wave
// of each group sits on every SIMD. Stage j is computed in phase j: its group issues only
// the stage's 32 MFMAs per wave (fragments already in registers) while the other group
// reads stage j + 1's fragments from LDS and issues the copies of stage j + 3. Three LDS
// buffers give the copies two phases to land. At the end group 1's int32 sums are added
// to group 0's through LDS (exact) and group 0 writes the tile.
template <int YMODE>
__device__ __forceinline__ void gemm_tile_ks(const int8_t* __restrict__ A, const float* __restrict__ xs,
                                             const int8_t* __restrict__ B, const float* __restrict__ ws,
                                             const float* __restrict__ bias, void* __restrict__ Y,
                                             int M, int N, int K, int m0, int n0, int8_t* smem) {
    constexpr int BM = 128, BN = 256, BKL = 128;
    constexpr int WM = 64, WN = 128, FM = WM / 32, FN = WN / 32;
    constexpr int STAGE_A = BM * BKL, STAGE = (BM + BN) * BKL;
    constexpr int CA = BM / 32, CB = BN / 32;   // copies of A and B per wave of a group (8 rows each)
    static_assert(3 * STAGE <= RING_BYTES, "three stages fit the LDS allocation");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm = q & 1, wn = q >> 1;
    const int KT = K / BKL;

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
    auto copies = [&](int kt) {
        int8_t* st = smem + (kt % 3) * STAGE;
        const int kc = min(kt, KT - 1);
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int so = __builtin_amdgcn_readfirstlane(kc * BKL + 8 * c * K);
            lds_copy16_buf(ra, cra + 8 * c < rows_a ? ((c & 1) ? va1 : va0) : 0x7FFFFFF0, so,
                           st + ((BM / 4) * q + 8 * c) * BKL);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int so = __builtin_amdgcn_readfirstlane(kc * BKL + 8 * c * K);
            lds_copy16_buf(rb, crb + 8 * c < rows_b ? ((c & 1) ? vb1 : vb0) : 0x7FFFFFF0, so,
                           st + STAGE_A + ((BN / 4) * q + 8 * c) * BKL);
        }
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    const int lr = lane & 31;
    const int fa_base = wm * WM * BKL + lr * BKL, fb_base = STAGE_A + wn * WN * BKL + lr * BKL;
    i32x4 F[4][FM + FN];
    auto read_stage = [&](int kt) {
        const int8_t* st = smem + (kt % 3) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int co = ((2 * ks + (lane >> 5)) ^ h128(lr)) << 4;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                F[ks][FM + j] = *reinterpret_cast<const i32x4*>(st + fb_base + co + j * 32 * BKL);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                F[ks][i] = *reinterpret_cast<const i32x4*>(st + fa_base + co + i * 32 * BKL);
        }
    };
    auto mfma_stage = [&]() {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F[ks][i], F[ks][FM + j], acc[i][j], 0, 0, 0);
    };
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int LGKM0 = vmcnt_le(63) & ~(0xF << 8);   // lgkmcnt(0), vmcnt left alone

    // Prologue: group 0 copies stages 0 and 2, group 1 stage 1 (stage 2 is needed in phase
    // 1, before any phase-0 copy could land); group 0 reads stage 0.
    if constexpr (YMODE != Y_I32)
        issue_scales(xs, ws, bias, M, N, m0, n0, wave, lane, smem);
    if (grp == 0) {
        copies(0);
        copies(2);   // past the end: a repeat of the last stage, never read
        __builtin_amdgcn_s_waitcnt(vmcnt_le(CA + CB) & ~(0xF << 8));   // stage 0 landed
    } else {
        copies(1);
    }
    phase_end();
    // Phase j: group (j & 1) runs stage j's MFMAs and then waits for the copies it issued
    // in phase j - 1 (stage j + 2); the other group issues stage j + 3's copies into stage
    // j's buffer (read in phase j - 1) and reads stage j + 1. Every wave runs the same
    // barriers (one per phase). Before phase 0 group 0 reads stage 0 while group 1 waits
    // for its stage-1 copies.
    // Each group runs its own straight-line loop over pairs of phases (a branch per phase
    // inside one loop would make the compiler keep two copies of the fragments).
    auto mfma_phase = [&]() {
        mfma_stage();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
        phase_end();
    };
    auto read_phase = [&](int j) {
        copies(j + 3);
        read_stage(min(j + 1, KT - 1));   // past the end: a repeat, never used
        __builtin_amdgcn_s_waitcnt(LGKM0);
        phase_end();
    };
    if (grp == 0) {
        read_stage(0);
        __builtin_amdgcn_s_waitcnt(LGKM0);
        phase_end();
        int j = 0;
        for (; j + 1 < KT; j += 2) {
            mfma_phase();        // phase j
            read_phase(j + 1);   // phase j + 1
        }
        if (j < KT)
            mfma_phase();
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));   // stage 1 landed
        phase_end();
        int j = 0;
        for (; j + 1 < KT; j += 2) {
            read_phase(j);       // phase j
            mfma_phase();        // phase j + 1
        }
        if (j < KT)
            read_phase(j);
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
                        i32x4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
    }
    phase_end();
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const i32x4 v = *reinterpret_cast<const i32x4*>(xch + ((i * FN + j) * 4 + e4) * 256 + lane * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][4 * e4 + r] += v[r];
                }
    }
    __builtin_amdgcn_s_waitcnt(LGKM0);
    if (grp == 0) {
        store_tile<WM, WN, FM, FN, YMODE, 4>(acc, bias != nullptr, Y, M, N, m0 + wm * WM, n0 + wn * WN,
                                             wm * WM, wn * WN, q, lane, smem);
    } else {
        barrier_no_fence();   // the one barrier store_tile runs
    }
}

// Tiles: the first `nbig` workgroups take 256 x 256 tiles of the first `nbig / tiles_m`
// N-panels; the rest take 128 x 256 tiles of the remaining panels. With 256 CUs, whole
// rounds of big tiles keep every CU busy and the leftover panels run as half-height
// tiles in a shorter final round. Within each group, workgroups are dealt to XCDs so
// that an XCD's tiles are consecutive and share W panels (column-major tile order).
struct TilePlan {
    int tiles_m_big, nbig, tiles_m_small, nsmall, n_small0;
};

// K % 128 == 0 runs 8 waves (2 x 4) per workgroup on the 128-byte path; other K run 4
// waves (2 x 2) on the 64-byte ring.
template <int YMODE, bool K128, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int K, TilePlan plan) {
    static_assert(K128 || NWV == 4, "the 64-byte ring runs 4 waves");
    constexpr int WGM = 2, WGN = NWV / 2;
    __shared__ __attribute__((aligned(1024))) int8_t smem[RING_BYTES + SCALE_BYTES];
    const int bid = blockIdx.x;
    if (bid < plan.nbig) {
        const int tile = xcd_remap(bid, plan.nbig);
        const int tn = tile / plan.tiles_m_big, tm = tile - tn * plan.tiles_m_big;
        if constexpr (K128 && NWV == 8 && GEMM_PINGPONG)
            gemm_tile_pp<256, 256, YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 256, tn * 256, smem);
        else if constexpr (K128)
            gemm_tile128<256, 256, WGM, WGN, YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 256, tn * 256, smem);
        else
            gemm_tile<256, 256, 4, YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 256, tn * 256, smem);
    } else {
        const int tile = xcd_remap(bid - plan.nbig, plan.nsmall);
        const int tn = tile / plan.tiles_m_small, tm = tile - tn * plan.tiles_m_small;
        if constexpr (K128 && NWV == 8 && GEMM_PINGPONG)
            gemm_tile_ks<YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 128, plan.n_small0 + tn * 256, smem);
        else if constexpr (K128)
            gemm_tile128<128, 256, WGM, WGN, YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 128,
                                                    plan.n_small0 + tn * 256, smem);
        else
            gemm_tile<128, 256, 5, YMODE>(A, xs, B, ws, bias, Y, M, N, K, tm * 128,
                                          plan.n_small0 + tn * 256, smem);
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

TilePlan plan_tiles(int64_t M, int64_t N) {
    TilePlan p{};
    const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
    const int total = tm * tn, cus = cu_count();
    int small_panels = 0;
    if (M <= 128) {
        small_panels = tn;                      // every tile is half height
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
    return p;
}

}  // namespace

ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0)
        return QL_OK;
    const TilePlan plan = plan_tiles(M, N);
    const dim3 grid((unsigned)(plan.nbig + plan.nsmall));
    const int m = (int)M, n = (int)N, k = (int)K;
#define QL_LAUNCH(MODE, K128)                                                                   \
    hipLaunchKernelGGL((gemm_w8a8_kernel<MODE, K128, K128 ? GEMM_WAVES_K128 : 4>), grid,          \
                       dim3(64 * (K128 ? GEMM_WAVES_K128 : 4)), 0, stream, xq, x_scale, wq,        \
                       w_scale, bias, y, m, n, k, plan)
    const bool k128 = K % 128 == 0;
    switch (y_mode) {
    case Y_F32:
        if (k128) QL_LAUNCH(Y_F32, true); else QL_LAUNCH(Y_F32, false);
        break;
    case Y_F16:
        if (k128) QL_LAUNCH(Y_F16, true); else QL_LAUNCH(Y_F16, false);
        break;
    default:
        if (k128) QL_LAUNCH(Y_I32, true); else QL_LAUNCH(Y_I32, false);
        break;
    }
#undef QL_LAUNCH
    return launch_status();
}

}  // namespace ql
