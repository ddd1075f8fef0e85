/*
 * nvfp4_oracle.h -- CPU oracle for NVFP4 quantization and the dequantize-then-matmul GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call this:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Conventions: x inputs are either IEEE fp32 (dtype 0) or bfloat16 bit patterns (dtype 1),
 * row-major [M][ld] with ld >= K.  packed is [M][K/2] (element 2i in the low nibble of byte i),
 * scales is [M][K/16] E4M3 bytes, S is the fp32 per-tensor scale.
 * Functions returning int give 0 on success, -1 when a documented precondition fails
 * (non-finite input, K not a multiple of 16, S not a finite positive number where one is needed).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double ora_e2m1_value(int code);                 /* value of a 4-bit E2M1 code (bit 3 = sign) */
double ora_e4m3_value(int byte);                 /* value of an OCP E4M3FN byte (NaN for 0x7F/0xFF) */
uint16_t ora_bf16_round(float y);                /* nearest bfloat16 (ties to even) of an fp32 value */

/* Dynamic per-tensor scale: S = RN32(max|x| / (6 * 448)). */
int ora_tensor_scale(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float *S);

/* Block scale byte for a 16-value block with amax = max|v| under tensor scale S. */
int ora_block_scale_byte(double amax, float S);

/* 4-bit code of one value v in a block whose scale byte is `byte`, under tensor scale S. */
int ora_element_code(float v, int byte, float S);

/* Full quantizer with a given tensor scale S (static mode; dynamic = ora_tensor_scale first). */
int ora_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float S,
                 uint8_t *packed, uint8_t *scales, int nthreads);

/* Dequantize to fp32 and/or bf16 ([M][K] each; either pointer may be NULL). */
int ora_dequantize(const uint8_t *packed, const uint8_t *scales, float S, int64_t M, int64_t K,
                   float *y_f32, uint16_t *y_bf16, int nthreads);

/* The same with block size b in {1, 2, 4, 8, 16, 32, 64} (K % b == 0, K even): one E4M3 byte per
   b consecutive values along K, scales [M][K/b] [NVFP4-DiT page, Algorithm 1 / Eq. 9 block sizes]. */
int ora_quantize_bs(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float S, int b,
                    uint8_t *packed, uint8_t *scales, int nthreads);
int ora_dequantize_bs(const uint8_t *packed, const uint8_t *scales, float S, int64_t M, int64_t K, int b,
                      float *y_f32, uint16_t *y_bf16, int nthreads);

/* MXFP4 (OCP microscaling): 32-value blocks, E8M0 scale X = 2^(floor(log2 amax) - 2), no tensor
   scale; scales are [M][K/32] bytes. */
int ora_mx_scale_byte(double amax);
int ora_mx_element_code(float v, int byte);
int ora_mx_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, uint8_t *packed,
                    uint8_t *scales, int nthreads);
int ora_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, float *y_f32,
                      uint16_t *y_bf16, int nthreads);

/* Y[i][j] = sum_k A[i][k]*B[j][k] accumulated in fp64; R[i][j] = sum_k |A[i][k]*B[j][k]|. */
int ora_gemm(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
             double *Y, double *R, int nthreads);

/* Same as ora_gemm for n chosen output elements (rows[t], cols[t]). */
int ora_gemm_sampled(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t K,
                     const int64_t *rows, const int64_t *cols, int64_t n, double *Y, double *R);

#ifdef __cplusplus
}
#endif
#endif
