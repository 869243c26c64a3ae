/*
 * ql_probe.h -- measurement probes (libqlprobe.so), not part of the quantized linear layer.
 *
 * The benchmark reports each kernel against the published MI355X peaks and also against
 * ceilings measured on the GPU at hand with these probes: the int8 matrix-core rate with no
 * memory traffic (for the W8A8 GEMM) and the rate at which one launch reads a buffer of a
 * given size from HBM (for the memory-bound kernels).
 *
 * Every pointer is a device pointer owned by the caller; work goes on `stream` (a
 * hipStream_t, NULL = the null stream) and the calls return without waiting. Each returns
 * 0 on success, -1 for a bad argument (nothing launched), or the HIP error code of the
 * launch.
 */
#ifndef QL_PROBE_H
#define QL_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of compute units of the current device, or -1. */
int qlp_cu_count(void);

/*
 * One workgroup of 256 threads per CU; each wave issues `iters` x 16 independent
 * v_mfma_i32_32x32x32_i8 (65536 int8 operations each) from registers. random_operands != 0
 * uses random bytes, 0 a constant pattern. sink: int32 [CUs * 256], written once per thread.
 * Operations per launch: CUs * 4 * iters * 16 * 65536.
 */
int qlp_mfma_i8(int64_t iters, int random_operands, int32_t* sink, void* stream);

/*
 * The same loop with operands loaded once from two code arrays of w_bytes and x_bytes bytes
 * (device pointers, 16-byte aligned, sizes multiples of 16, at least 16): lane t's four
 * 16-byte fragments are the array's 16-byte pieces 4 t .. 4 t + 3 (wrapping around), W's the
 * matrix core's first operand. Returns -1 on a bad argument. Same sink and operation count.
 */
int qlp_mfma_i8_data(int64_t iters, const int8_t* w, int64_t w_bytes, const int8_t* x, int64_t x_bytes,
                     int32_t* sink, void* stream);

/*
 * Reads `bytes` bytes at `src` once (bytes % 16 == 0, src 16-byte aligned), one workgroup of
 * 8 waves per CU. sink: uint32 [CUs * 512], written once per thread.
 */
int qlp_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QL_PROBE_H */
