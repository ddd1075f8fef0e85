/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 block-scaled 4-bit quantization and the
 * dequantize-then-matmul GEMM.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the benchmark's
 * CPU-baseline leg.  It shares no code with the HIP library and the library never calls it.
 *
 * What it computes (sources are the pages this project follows):
 *
 *  * Element format E2M1 [NVFP4-DiT page, Methodology section 1, text after Definition III.1]:
 *    1 sign, 2 exponent and 1 mantissa bit.  With exponent field E and mantissa bit m the
 *    magnitude is m/2 when E = 0 and 2^(E-1) * (1 + m/2) otherwise, i.e. the grid
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  (The page's printed magnitude list contains 0.75 and omits 0;
 *    we read that as a garble and follow the bit format.)
 *
 *  * Quantizer Q_FP4(v; s) = s * clip(round(v / s)_FP4, -6, 6) [NVFP4-DiT page, Definition III.1].
 *    The page leaves the rounding rule open; we read round(.)_FP4 as round-to-nearest on the
 *    E2M1 grid with ties to the even code, evaluated on the exact real quotient v/s.
 *    Nearest-on-the-finite-grid already saturates at +-6, so the clip is implied.
 *
 *  * Two-level scale [vllm-omni RFC "NVFP4 Quantization Support for Diffusion Models",
 *    Motivation]: one FP8 scale per 16 consecutive values and one FP32 scale per tensor, so the
 *    block scale of Definition III.1 is s = e * S with e an E4M3 value and S the fp32 tensor scale.
 *    The pages do not say how e and S are chosen.  Our reading:
 *      - S (dynamic) = RN32(amax_tensor / (6 * 448)): the tensor maximum lands on the top of both
 *        grids; one IEEE fp32 division.  S (static) is given by the caller.
 *      - e = the E4M3 value nearest to amax_block / (6 S) (ties to the even byte), saturating at
 *        448, so the block maximum lands near 6 on the E2M1 grid.  e = 0 (byte 0x00) when the
 *        block is all zeros or the ratio rounds to zero; such a block quantizes to magnitude 0.
 *      - E4M3 is the OCP "FN" variant: bias 7, subnormals k * 2^-9, max 0x7E = 448, no infinity,
 *        0x7F/0xFF are NaN and never produced.
 *      - The sign bit of every code copies the sign bit of the input (so -0.0 and negative
 *        values that round to zero give code 8).
 *
 *  * Packing [NVFP4-DiT page, Methodology section 3 "Systems optimization"]: two FP4 codes per
 *    byte; the order is unstated, we put element 2i in the low nibble of byte i.
 *
 *  * Dequantize: y = RN32(sign * q * e * S), one rounding of the exact product; bf16 output is
 *    the nearest bfloat16 (ties to even) of that fp32 value.
 *
 *  * GEMM [NVFP4-DiT page, Methodology section 3: on-the-fly dequantization, FP32
 *    accumulation]: Y = dequant(A) * dequant(B)^T with fp32 operands, accumulated here in fp64
 *    so that the oracle's own rounding is far below the comparison tolerance; R = sum |a*b| is
 *    returned alongside for the per-element tolerance.
 *
 * Exactness of the decisions.  Every rounding decision is made by comparing distances
 * |a - P| between the input magnitude a (an fp32 value, <= 24 significant bits) and candidate
 * points P = g * e * S or P = v_e4m3 * 6 * S.  Each P is a product of a value with <= 5 significant
 * bits, a value with <= 4 significant bits and S (24 bits), so it has <= 31 significant bits and is
 * exact in fp64.  For the two candidates adjacent to a, a - P spans <= 32 bits and is exact too, so
 * ties are seen as exact ties and every other comparison is strict; farther candidates are at
 * least one grid gap away, which fp64 rounding cannot close.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element and scale formats ---------------------------------------------------------- */

double ora_e2m1_value(int code) {
  int sign = (code >> 3) & 1, E = (code >> 1) & 3, m = code & 1;
  double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
  return sign ? -mag : mag;
}

double ora_e4m3_value(int byte) {
  int sign = (byte >> 7) & 1, E = (byte >> 3) & 15, m = byte & 7;
  double mag;
  if (E == 15 && m == 7) return NAN;
  if (E == 0) mag = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
  else mag = ldexp(1.0 + m / 8.0, E - 7);
  return sign ? -mag : mag;
}

static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float load_x(const void *x, int dtype, int64_t idx) {
  if (dtype == 0) return ((const float *)x)[idx];
  return bf16_bits_to_float(((const uint16_t *)x)[idx]);
}

uint16_t ora_bf16_round(float y) {
  /* The two bfloat16 neighbours of y are its truncation and the next one away from zero;
     pick the nearer, ties to the even pattern. */
  uint32_t u;
  memcpy(&u, &y, 4);
  if (isnan(y)) return (uint16_t)((u >> 16) | 0x40);
  uint16_t lo = (uint16_t)(u >> 16), hi = (uint16_t)(lo + 1);
  if (isinf(y)) return lo;
  /* Above the largest finite bfloat16 the next step would be 2^128; reaching half of it
     overflows to infinity, whose pattern is exactly lo + 1. */
  double vhi = ((lo & 0x7FFF) == 0x7F7F) ? copysign(ldexp(1.0, 128), (double)y)
                                         : (double)bf16_bits_to_float(hi);
  double dlo = fabs((double)y - (double)bf16_bits_to_float(lo));
  double dhi = fabs(vhi - (double)y);
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1) ? hi : lo;
}

/* ---- tensor scale ------------------------------------------------------------------------ */

int ora_tensor_scale(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float *S) {
  float amax = 0.0f;
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) {
      float v = load_x(x, dtype, i * ld + k);
      if (!isfinite(v)) return -1;
      if (fabsf(v) > amax) amax = fabsf(v);
    }
  *S = amax / 2688.0f; /* 2688 = 6 * 448; one correctly rounded fp32 division */
  return 0;
}

/* ---- block scale and element codes ------------------------------------------------------- */

int ora_block_scale_byte(double amax, float S) {
  if (amax == 0.0) return 0;
  /* nearest E4M3 value to amax / (6 S): compare amax with every candidate v * 6 * S */
  double six_s = 6.0 * (double)S;
  int best = 0;
  double best_d = INFINITY;
  for (int b = 0; b <= 0x7E; ++b) {
    double d = fabs(amax - ora_e4m3_value(b) * six_s);
    if (d < best_d || (d == best_d && (b & 1) == 0)) {
      best = b;
      best_d = d;
    }
  }
  return best;
}

int ora_element_code(float v, int byte, float S) {
  int sign = signbit(v) ? 8 : 0;
  double e = ora_e4m3_value(byte);
  if (e == 0.0) return sign; /* flushed block */
  double es = e * (double)S;
  double a = fabs((double)v);
  int best = 0;
  double best_d = INFINITY;
  for (int m = 0; m < 8; ++m) {
    double d = fabs(a - ora_e2m1_value(m) * es);
    if (d < best_d || (d == best_d && (m & 1) == 0)) {
      best = m;
      best_d = d;
    }
  }
  return sign | best;
}

/* ---- quantize / dequantize ---------------------------------------------------------------- */

/* Block size b (the page's Algorithm 1 / Eq. 9 chooses b from {1, 2, 4, 8, 16, 32, 64} per layer;
   the format is otherwise unchanged): every run of b consecutive values along K has one E4M3 byte.
   scales is [M][K/b]. */
static int valid_block(int64_t K, int b) {
  return (b == 1 || b == 2 || b == 4 || b == 8 || b == 16 || b == 32 || b == 64) && K % b == 0 && K % 2 == 0;
}

int ora_quantize_bs(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float S, int b,
                    uint8_t *packed, uint8_t *scales, int nthreads) {
  if (!valid_block(K, b) || ld < K || !(S >= 0.0f) || !isfinite(S)) return -1;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16) reduction(| : bad)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < K / b; ++j) {
      double amax = 0.0;
      for (int t = 0; t < b; ++t) {
        float v = load_x(x, dtype, i * ld + b * j + t);
        if (!isfinite(v)) bad = 1;
        if (fabs((double)v) > amax) amax = fabs((double)v);
      }
      if (amax > 0.0 && S == 0.0f) bad = 1;
      int byte = (amax > 0.0 && S > 0.0f) ? ora_block_scale_byte(amax, S) : 0;
      scales[i * (K / b) + j] = (uint8_t)byte;
      for (int t = 0; t < b; ++t) {
        int64_t k = b * j + t;
        int c = ora_element_code(load_x(x, dtype, i * ld + k), byte, S);
        uint8_t *dst = &packed[i * (K / 2) + k / 2];
        if (k & 1) *dst = (uint8_t)((*dst & 0x0F) | (c << 4));
        else *dst = (uint8_t)((*dst & 0xF0) | c);
      }
    }
  }
  return bad ? -1 : 0;
}

int ora_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, float S,
                 uint8_t *packed, uint8_t *scales, int nthreads) {
  if (K % 16 != 0) return -1;
  return ora_quantize_bs(x, dtype, M, K, ld, S, 16, packed, scales, nthreads);
}

int ora_dequantize_bs(const uint8_t *packed, const uint8_t *scales, float S, int64_t M, int64_t K, int b,
                      float *y_f32, uint16_t *y_bf16, int nthreads) {
  if (!valid_block(K, b) || !isfinite(S)) return -1;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16) reduction(| : bad)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t k = 0; k < K; ++k) {
      int byte = scales[i * (K / b) + k / b];
      if ((byte & 0x7F) == 0x7F) bad = 1;
      int code = (packed[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
      double exact = ora_e2m1_value(code) * ora_e4m3_value(byte) * (double)S;
      float y = (float)exact; /* the product is exact in fp64: this is the single rounding */
      if (y_f32) y_f32[i * K + k] = y;
      if (y_bf16) y_bf16[i * K + k] = ora_bf16_round(y);
    }
  }
  return bad ? -1 : 0;
}

int ora_dequantize(const uint8_t *packed, const uint8_t *scales, float S, int64_t M, int64_t K,
                   float *y_f32, uint16_t *y_bf16, int nthreads) {
  if (K % 16 != 0) return -1;
  return ora_dequantize_bs(packed, scales, S, M, K, 16, y_f32, y_bf16, nthreads);
}

/* ---- MXFP4 ---------------------------------------------------------------------------------
 *
 * The vllm-omni RFC (Motivation) names MXFP4 as the related microscaling format but does not
 * define it; these functions follow the public OCP Microscaling (MX) format definition:
 *   - blocks of 32 consecutive values along K share one E8M0 scale X = 2^(b - 127), b a byte
 *     (255 would be NaN and is never produced);
 *   - X = 2^(floor(log2 amax) - 2), 2 being the largest E2M1 exponent, so amax / X lies in
 *     [4, 8); b is clamped to [0, 254], and an all-zero block gets b = 0;
 *   - each value becomes the E2M1 value nearest to v / X (ties to the even code, clipped to +-6),
 *     sign bit copied; there is no per-tensor scale;
 *   - dequantize: y = RN32(q * X), which is exact for every scale byte the quantizer produces
 *     from finite fp32 / bf16 input (b <= 252); larger bytes can round to +-inf.
 * Packing is the same as NVFP4 (element 2i in the low nibble of byte i); scales are [M][K/32].
 */
int ora_mx_scale_byte(double amax) {
  if (amax == 0.0) return 0;
  int e;
  (void)frexp(amax, &e); /* amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
  int b = (e - 1) - 2 + 127;
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

int ora_mx_element_code(float v, int byte) {
  double X = ldexp(1.0, byte - 127);
  double a = fabs((double)v);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 8; ++c) { /* nearest of the 8 magnitudes; on a tie keep the even code */
    double d = fabs(a - ora_e2m1_value(c) * X);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best | (signbit(v) ? 8 : 0);
}

int ora_mx_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, uint8_t *packed,
                    uint8_t *scales, int nthreads) {
  if (K % 32 != 0 || ld < K) return -1;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16) reduction(| : bad)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < K / 32; ++j) {
      float v[32];
      double amax = 0.0;
      for (int t = 0; t < 32; ++t) {
        v[t] = load_x(x, dtype, i * ld + 32 * j + t);
        if (!isfinite(v[t])) bad = 1;
        if (fabs((double)v[t]) > amax) amax = fabs((double)v[t]);
      }
      int byte = ora_mx_scale_byte(amax);
      scales[i * (K / 32) + j] = (uint8_t)byte;
      for (int t = 0; t < 32; t += 2) {
        int c0 = ora_mx_element_code(v[t], byte), c1 = ora_mx_element_code(v[t + 1], byte);
        packed[i * (K / 2) + 16 * j + t / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  }
  return bad ? -1 : 0;
}

int ora_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, float *y_f32,
                      uint16_t *y_bf16, int nthreads) {
  if (K % 32 != 0) return -1;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16) reduction(| : bad)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t k = 0; k < K; ++k) {
      int byte = scales[i * (K / 32) + k / 32];
      if (byte == 255) bad = 1;
      int code = (packed[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
      float y = (float)(ora_e2m1_value(code) * ldexp(1.0, byte - 127)); /* exact */
      if (y_f32) y_f32[i * K + k] = y;
      if (y_bf16) y_bf16[i * K + k] = ora_bf16_round(y);
    }
  }
  return bad ? -1 : 0;
}

/* ---- GEMM --------------------------------------------------------------------------------- */

int ora_gemm(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
             double *Y, double *R, int nthreads) {
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = (double)A[i * lda + k] * (double)B[j * ldb + k];
        acc += p;
        mag += fabs(p);
      }
      Y[i * N + j] = acc;
      if (R) R[i * N + j] = mag;
    }
  }
  return 0;
}

int ora_gemm_sampled(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t K,
                     const int64_t *rows, const int64_t *cols, int64_t n, double *Y, double *R) {
  for (int64_t t = 0; t < n; ++t) {
    double acc = 0.0, mag = 0.0;
    const float *a = A + rows[t] * lda, *b = B + cols[t] * ldb;
    for (int64_t k = 0; k < K; ++k) {
      double p = (double)a[k] * (double)b[k];
      acc += p;
      mag += fabs(p);
    }
    Y[t] = acc;
    if (R) R[t] = mag;
  }
  return 0;
}
