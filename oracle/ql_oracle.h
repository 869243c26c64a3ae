/* ql_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * The oracle's own header: nothing in the HIP library includes it. */
#ifndef QL_ORACLE_H
#define QL_ORACLE_H
#include <stdint.h>

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float x);
void oracle_f16_to_f32_array(const uint16_t* h, int64_t n, float* out);
void oracle_f32_to_f16_array(const float* x, int64_t n, uint16_t* out);

void oracle_quant_rows_i8(const float* x, int64_t rows, int64_t cols, int8_t* q, float* scale);
float oracle_quant_tensor_i8(const float* x, int64_t n, int8_t* q);

int oracle_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                    int32_t* acc);
void oracle_epilogue_w8a8(const int32_t* acc, const float* x_scale, const float* w_scale,
                          const float* bias, int64_t M, int64_t N, float* y32, double* y64);

void oracle_wonly_f64(const float* x, int64_t M, int64_t K, const void* codes, int codes_kind,
                      const float* scale, const uint8_t* zp, int64_t group, const float* bias,
                      int64_t N, double* y64);
void oracle_w4a16_f64(const float* x, int64_t M, int64_t K, const int32_t* packed,
                      const uint16_t* scale16, int64_t group, const float* bias, int64_t N,
                      double* y64);
void oracle_unpack_int4(const int32_t* packed, int64_t N, int64_t K, int8_t* q);

void oracle_quant_block_asym_u8(const float* w, int64_t N, int64_t K, int64_t block,
                                uint8_t* q, float* scale, uint8_t* zp);
void oracle_quant_int4_group(const float* w, int64_t N, int64_t K, int64_t group,
                             int32_t* packed, uint16_t* scale16);

void oracle_activation_f64(double* y, int64_t n, int act);
double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float x);
void oracle_quant_rows_e4m3(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale);
void oracle_gemm_e4m3_f64(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                          const float* w_scale, const float* bias, int64_t M, int64_t N,
                          int64_t K, double* y64, double* mag);
void oracle_quant_rows_i8_asym(const float* x, int64_t rows, int64_t cols, int8_t* q,
                               float* scale, float* zero);
void oracle_column_sums_i8(const int8_t* wq, int64_t N, int64_t K, int32_t* colsum);
void oracle_w8a8_asym_f64(const int8_t* xq, const float* x_scale, const float* x_zero,
                          const int8_t* wq, const float* w_scale, const float* bias, int64_t M,
                          int64_t N, int64_t K, double* y64);
int oracle_num_threads(void);

void oracle_channel_scales(const float* y, int64_t M, int64_t N, float* s);
void oracle_requant_i8(const float* y, int64_t M, int64_t N, const float* s, int64_t scale_n,
                       int8_t* q);
void oracle_wonly_f32seq(const float* x, int64_t M, int64_t K, const void* codes, int codes_kind,
                         const float* scale, const uint8_t* zp, int64_t group, const float* bias,
                         int64_t N, float* y32);
#endif
