/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every entry point on small
 * inputs that reach its edge cases (signed zeros, all-zero and tiny blocks, values far above
 * 448 * 6 * S, exact ties, every block size, MXFP4, the sampled GEMM), with a few invariants checked
 * (codes within the format, scale bytes never 0x7F, the GEMM's R bounding |Y|).  The oracle is test
 * infrastructure; this driver is its memory- and UB-safety check.  Exit 0 = clean run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

static int failures = 0;
#define EXPECT(cond)                                                                            \
  do {                                                                                          \
    if (!(cond)) {                                                                              \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond);           \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64 in [0, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) * 0x1p-53;
}

static uint16_t to_bf16(float f) { return ora_bf16_round(f); }

int main(void) {
  enum { M = 37, K = 192, N = 29 };
  static float x[M * (K + 16)];
  static uint16_t xb[M * K];
  for (int i = 0; i < M * (K + 16); ++i) x[i] = (float)((urand() - 0.5) * ldexp(1.0, (int)(urand() * 40) - 20));
  for (int j = 0; j < 16; ++j) x[j] = 0.0f;                      /* an all-zero block */
  for (int j = 16; j < 32; ++j) x[j] = -0.0f;                    /* negative zeros */
  for (int j = 32; j < 48; ++j) x[j] = 1e-30f * (float)(j - 40);  /* a tiny block */
  x[50] = 3.0e4f;                                                 /* far above the others */
  for (int i = 0; i < M * K; ++i) xb[i] = to_bf16(x[i]);

  for (int c = 0; c < 16; ++c) EXPECT(fabs(ora_e2m1_value(c)) <= 6.0);
  for (int b = 0; b < 256; ++b) (void)ora_e4m3_value(b);
  float S = 0.0f;
  EXPECT(ora_tensor_scale(x, 0, M, K, K + 16, &S) == 0 && S > 0.0f);
  EXPECT(ora_tensor_scale(xb, 1, M, K, K, &S) == 0 && S > 0.0f);
  const float scales_S[] = {S, 0x1p-8f, 1.1f * 0x1p-9f, 0x1p-120f, 0x1p100f};
  static uint8_t packed[M * K / 2], sc[M * K], packed2[M * K / 2], sc2[M * K];
  static float y32[M * K];
  static uint16_t y16[M * K];
  for (unsigned t = 0; t < sizeof(scales_S) / sizeof(scales_S[0]); ++t) {
    const float St = scales_S[t];
    EXPECT(ora_quantize(x, 0, M, K, K + 16, St, packed, sc, 2) == 0);
    EXPECT(ora_quantize(xb, 1, M, K, K, St, packed2, sc2, 1) == 0);
    for (int i = 0; i < M * K / 16; ++i) EXPECT(sc[i] <= 0x7E && sc2[i] <= 0x7E);
    EXPECT(ora_dequantize(packed, sc, St, M, K, y32, y16, 2) == 0);
    EXPECT(ora_dequantize(packed, sc, St, M, K, NULL, y16, 1) == 0);
    for (int b = 1; b <= 64; b *= 2) {
      EXPECT(ora_quantize_bs(x, 0, M, K, K + 16, St, b, packed2, sc2, 2) == 0);
      EXPECT(ora_dequantize_bs(packed2, sc2, St, M, K, b, y32, NULL, 1) == 0);
    }
    for (int i = 0; i < 64; ++i) {
      const int byte = ora_block_scale_byte(fabs((double)x[i]), St);
      EXPECT(byte >= 0 && byte <= 0x7E);
      EXPECT(ora_element_code(x[i], byte, St) >= 0 && ora_element_code(x[i], byte, St) < 16);
    }
  }
  /* preconditions: non-finite input and an invalid static scale are reported, not read past */
  const float bad = NAN;
  float xn[32];
  memcpy(xn, x, sizeof xn);
  xn[7] = bad;
  EXPECT(ora_quantize(xn, 0, 1, 32, 32, 1.0f, packed, sc, 1) != 0);
  EXPECT(ora_quantize(x, 0, 1, 32, 32, -1.0f, packed, sc, 1) != 0);
  EXPECT(ora_quantize(x, 0, 1, 24, 24, 1.0f, packed, sc, 1) != 0);

  /* MXFP4 */
  static uint8_t mp[M * K / 2], ms[M * K / 32];
  EXPECT(ora_mx_quantize(x, 0, M, K, K + 16, mp, ms, 2) == 0);
  EXPECT(ora_mx_dequantize(mp, ms, M, K, y32, y16, 2) == 0);
  for (int i = 0; i < 64; ++i) (void)ora_mx_element_code(x[i], ora_mx_scale_byte(fabs((double)x[i])));

  /* GEMM, full and sampled */
  static float A[M * K], B[N * K];
  static double Y[M * N], R[M * N], Ys[8], Rs[8];
  for (int i = 0; i < M * K; ++i) A[i] = (float)(urand() - 0.5);
  for (int i = 0; i < N * K; ++i) B[i] = (float)(urand() - 0.5);
  EXPECT(ora_gemm(A, K, B, K, M, N, K, Y, R, 3) == 0);
  for (int i = 0; i < M * N; ++i) EXPECT(fabs(Y[i]) <= R[i]);
  const int64_t rows[8] = {0, 1, 5, 36, 36, 0, 17, 9}, cols[8] = {0, 28, 3, 0, 28, 13, 1, 9};
  EXPECT(ora_gemm_sampled(A, K, B, K, K, rows, cols, 8, Ys, Rs) == 0);
  for (int t = 0; t < 8; ++t) EXPECT(Ys[t] == Y[rows[t] * N + cols[t]] && Rs[t] == R[rows[t] * N + cols[t]]);

  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("oracle driver ok\n");
  return failures ? 1 : 0;
}
