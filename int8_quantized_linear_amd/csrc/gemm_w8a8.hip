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
// Tile: 256 (M) x 256 (N) per workgroup of 4 waves (2 x 2); each wave owns a 128 x 128
// block of accumulators = 8 x 8 v_mfma_i32_16x16x64_i8 tiles (256 accumulator registers
// per lane). K advances 64 bytes per step through a ring of 4 LDS stages that global ->
// LDS direct loads (no register staging) fill three steps ahead; each step reads the
// next step's MFMA fragments while its own MFMAs run, with one barrier per step.
#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BK = 64;
constexpr int NTHR = 256;

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

// Tile geometry: BM x BN outputs per workgroup of 4 waves laid out 2 x 2, each wave
// WM x WN = (BM/2) x (BN/2); STAGES LDS buffers of BK = 64 k-columns each.
template <int BM_, int BN_, int STAGES_>
struct Geo {
    static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_;
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int STAGE_A = BM * BK, STAGE = (BM + BN) * BK;
    static constexpr int LA = BM * BK / 16 / NTHR, LB = BN * BK / 16 / NTHR;  // copies/thread
    static constexpr int LOADS = LA + LB;
};

template <int BM_, int BN_, int STAGES_, int YMODE>
__global__ __launch_bounds__(NTHR, 2) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int K, int tiles_m, int tiles_n) {
    using G = Geo<BM_, BN_, STAGES_>;
    constexpr int BM = G::BM, BN = G::BN, STAGES = G::STAGES, WM = G::WM, WN = G::WN;
    constexpr int FM = G::FM, FN = G::FN, STAGE_A = G::STAGE_A, STAGE = G::STAGE;
    constexpr int LA = G::LA, LB = G::LB, LOADS = G::LOADS;
    __shared__ __attribute__((aligned(1024))) int8_t smem[STAGES * STAGE];

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m, tm = tile - tn * tiles_m;  // neighbours share the W panel
    const int m0 = tm * BM, n0 = tn * BN;
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

    i32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = i32x4{0, 0, 0, 0};

    // Fragment reads: lane l takes row (l & 15) of a 16-row block and logical chunk (l >> 4)
    // of the 64-byte k-step; A and B use the same k <-> (lane, byte) assignment, so their
    // products pair the same k. rowhash depends on the low 4 row bits only, so a wave's
    // blocks are one base address plus multiples of 1 KB.
    const int fa_off = swz(wm * WM + (lane & 15), lane >> 4);
    const int fb_off = STAGE_A + swz(wn * WN + (lane & 15), lane >> 4);
    auto read_frags = [&](int kt, i32x4 (&fa)[FM], i32x4 (&fb)[FN]) {
        const int8_t* st = smem + (kt % STAGES) * STAGE;
        // B first: the next step's first MFMAs use A block 0 with every B block
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[j] = *reinterpret_cast<const i32x4*>(st + fb_off + j * 16 * BK);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[i] = *reinterpret_cast<const i32x4*>(st + fa_off + i * 16 * BK);
    };
    auto mfmas = [&](const i32x4 (&fa)[FM], const i32x4 (&fb)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    // Step kt: wait until stage kt+1 has landed (only the copies of the stages after it
    // may still be pending), barrier, issue stage kt+STAGES-1 into the buffer that held
    // stage kt-1 (every wave consumed those fragments before the barrier), read stage
    // kt+1's fragments, and run stage kt's MFMAs with the copies and reads spread among
    // them. Past the last stage the copies repeat the last stage (the buffers they fill
    // are never read), so every step has the same shape. sched_barrier(0) keeps steps
    // from being interleaved with each other.
    constexpr int NMF = FM * FN, NDS = FM + FN;
    // Before step kt's wait, stages 0 .. kt+STAGES-2 have been issued.
    static_assert(STAGES >= 3, "the ring needs a buffer being read, one landing, one free");
    auto step = [&](int kt, const i32x4 (&fa)[FM], const i32x4 (&fb)[FN], i32x4 (&na)[FM],
                    i32x4 (&nb)[FN]) {
        __builtin_amdgcn_s_waitcnt(vmcnt_le((STAGES - 3) * LOADS));
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + STAGES - 1);
        read_frags(kt + 1, na, nb);
        mfmas(fa, fb);
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
    i32x4 f0a[FM], f0b[FN], f1a[FM], f1b[FN];
    int k0;
    if (KT & 1) {
        k0 = -1;
#pragma unroll
        for (int s = 0; s < STAGES - 2; ++s)
            issue(s);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f0a[i] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f0b[j] = i32x4{0, 0, 0, 0};
    } else {
        k0 = 0;
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            issue(s);
        __builtin_amdgcn_s_waitcnt(vmcnt_le((STAGES - 2) * LOADS));
        barrier_no_fence();
        read_frags(0, f0a, f0b);
    }
    for (int kt = k0; kt < KT; kt += 2) {
        step(kt, f0a, f0b, f1a, f1b);
        step(kt + 1, f1a, f1b, f0a, f0b);   // reads past the end on the last pair: unused
    }
    // No copy into LDS may still be in flight when the workgroup's LDS is released.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));

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

template <class G>
ql_status launch_geo(const int8_t* xq, const float* x_scale, const int8_t* wq,
                     const float* w_scale, const float* bias, void* y, int y_mode, int64_t M,
                     int64_t N, int64_t K, hipStream_t stream) {
    const int tiles_m = (int)((M + G::BM - 1) / G::BM), tiles_n = (int)((N + G::BN - 1) / G::BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(NTHR);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (y_mode) {
    case Y_F32:
        hipLaunchKernelGGL((gemm_w8a8_kernel<G::BM, G::BN, G::STAGES, Y_F32>), grid, block, 0, stream, xq, x_scale, wq,
                           w_scale, bias, y, m, n, k, tiles_m, tiles_n);
        break;
    case Y_F16:
        hipLaunchKernelGGL((gemm_w8a8_kernel<G::BM, G::BN, G::STAGES, Y_F16>), grid, block, 0, stream, xq, x_scale, wq,
                           w_scale, bias, y, m, n, k, tiles_m, tiles_n);
        break;
    default:
        hipLaunchKernelGGL((gemm_w8a8_kernel<G::BM, G::BN, G::STAGES, Y_I32>), grid, block, 0, stream, xq, x_scale, wq,
                           w_scale, bias, y, m, n, k, tiles_m, tiles_n);
        break;
    }
    return launch_status();
}

}  // namespace

ql_status launch_gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, int y_mode,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0)
        return QL_OK;
    return launch_geo<Geo<256, 128, 3>>(xq, x_scale, wq, w_scale, bias, y, y_mode, M, N, K,
                                        stream);
}

}  // namespace ql
