/* Host-side checks of libnvfp4's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built from the library's own sources with the sanitizers on host code only, and run on a machine
 * without a GPU: every call below either fails validation before any HIP call (fake, never
 * dereferenced device pointers) or reaches the device check, which reports NVFP4_ERR_HIP or
 * NVFP4_ERR_DEVICE there.  The size queries are driven with extreme arguments, where the 64-bit size
 * arithmetic must neither overflow nor return a size for an invalid call.  Exit status 0 = all
 * expectations held (the sanitizers abort on the first finding). */
#include <stdint.h>
#include <stdio.h>

#include "nvfp4.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

#define P ((void *)0x10000)
#define P8 ((void *)0x10008)
#define PODD ((void *)0x10001)
#define U8(p) ((uint8_t *)(p))
#define F(p) ((float *)(p))

static int device_or_hip(nvfp4_status_t s) { return s == NVFP4_ERR_HIP || s == NVFP4_ERR_DEVICE || s == NVFP4_OK; }

int main(void) {
  const int64_t big = (int64_t)1 << 62, huge = INT64_MAX;
  EXPECT(nvfp4_abi_version() == NVFP4_ABI_VERSION);
  for (int s = -1; s < 12; ++s) EXPECT(nvfp4_status_string((nvfp4_status_t)s) != NULL);
  /* debug checks: the switch returns the previous setting; validation still comes first */
  {
    const int prev = nvfp4_set_debug_checks(1);
    EXPECT(nvfp4_set_debug_checks(1) == 1);
    EXPECT(nvfp4_quantize(P, NVFP4_BF16, 4, 24, 32, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, 4096, NULL) ==
           NVFP4_ERR_SHAPE);
    EXPECT(device_or_hip(nvfp4_quantize(P, NVFP4_BF16, 4, 32, 32, U8(P), U8(P), F(P), NVFP4_SCALE_STATIC, NULL, 0,
                                        NULL)));
    EXPECT(nvfp4_set_debug_checks(prev) == 1);
  }

  /* size queries at the edges */
  EXPECT(nvfp4_prepacked_bytes(huge, 16) == 0);
  EXPECT(nvfp4_prepacked_bytes(16, huge) == 0);
  EXPECT(nvfp4_prepacked_bytes(-1, 128) == 0);
  EXPECT(nvfp4_prepacked_bytes(big, big) == 0);
  EXPECT(nvfp4_prepacked_bytes(1152, 1152) == 36u * 9u * 2304u);
  EXPECT(nvfp4_quantize_workspace_bytes(huge, huge) > 0);
  for (int mode = -1; mode < 3; ++mode) {
    EXPECT(nvfp4_gemm_workspace_bytes_ld((nvfp4_mode_t)mode, huge, huge, huge, huge) == 0);
    EXPECT(nvfp4_gemm_workspace_bytes_ld((nvfp4_mode_t)mode, 1, 16, 1 << 30, huge) == 0);
    EXPECT(nvfp4_gemm_requant_workspace_bytes_ld((nvfp4_mode_t)mode, big, 16, 128, 128) == 0);
    EXPECT(nvfp4_gemm_requant_workspace_bytes_ld((nvfp4_mode_t)mode, 1 << 20, 1 << 20, 1 << 20, 1 << 20) == 0);
    (void)nvfp4_gemm_workspace_bytes((nvfp4_mode_t)mode, 4096, 1152, 4608);
    (void)nvfp4_gemm_requant_workspace_bytes((nvfp4_mode_t)mode, 4096, 1152, 4608);
    for (int64_t M = 1; M <= 8192; M *= 8)
      for (int64_t N = 16; N <= 16384; N *= 4)
        for (int64_t K = 16; K <= 12288; K *= 3) {
          if (K % 16) continue;
          for (int64_t pad = 0; pad <= 144; pad += 16) {
            (void)nvfp4_gemm_workspace_bytes_ld((nvfp4_mode_t)mode, M, N, K, K + pad);
            (void)nvfp4_gemm_requant_workspace_bytes_ld((nvfp4_mode_t)mode, M, N, K, K + pad);
          }
        }
  }

  /* quantize / fake quantize / dequantize validation */
  const size_t qws = nvfp4_quantize_workspace_bytes(4, 32);
  EXPECT(nvfp4_quantize(P, NVFP4_BF16, 4, 32, 32, U8(P), U8(P), NULL, NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_quantize(P, NVFP4_BF16, huge, 32, 32, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize(P, NVFP4_BF16, big, big, big, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize(P, NVFP4_BF16, 4, 32, 16, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_STRIDE);
  EXPECT(nvfp4_quantize(PODD, NVFP4_BF16, 4, 32, 32, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_quantize(P, NVFP4_BF16, 4, 32, 32, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, NULL, 0, NULL) == NVFP4_ERR_WORKSPACE);
  EXPECT(device_or_hip(nvfp4_quantize(P, NVFP4_BF16, 4, 32, 32, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL)));
  EXPECT(nvfp4_quantize_bs(P, NVFP4_F32, 4, 48, 48, 32, U8(P), U8(P), F(P), NVFP4_SCALE_STATIC, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize_bs(P, NVFP4_F32, 4, 64, 64, 8, U8(P), U8(P), F(P), NVFP4_SCALE_STATIC, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize_noalloc(P, NVFP4_BF16, 4, 24, 24, 16, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(device_or_hip(nvfp4_quantize_noalloc(P, NVFP4_BF16, 4, 32, 32, 16, U8(P), U8(P), F(P), NVFP4_SCALE_DYNAMIC, NULL)));
  EXPECT(nvfp4_fake_quantize(P, NVFP4_BF16, 4, 32, 32, P8, NVFP4_F32, 32, F(P), NVFP4_SCALE_DYNAMIC, P, qws, NULL) == NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_dequantize(U8(P), U8(P), F(P), huge, 16, P, NVFP4_F32, 16, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_dequantize(U8(P), U8(P), F(P), 4, 32, P, (nvfp4_dtype_t)7, 32, NULL) == NVFP4_ERR_DTYPE);
  EXPECT(device_or_hip(nvfp4_dequantize(U8(P), U8(P), F(P), 4, 32, P, NVFP4_BF16, 32, NULL)));
  EXPECT(nvfp4_prepack_weight(U8(P), U8(P), huge, 128, P, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_unpack_weight_bs(P, 32, 128, 48, U8(P), U8(P), NULL) == NVFP4_ERR_SHAPE);

  /* GEMM validation, including the extents the kernels' 32-bit indices need */
  EXPECT(nvfp4_gemm(NVFP4_W4A4, P, U8(P), F(P), P, F(P), 1, 16, 1 << 30, 1 << 30, P, NVFP4_BF16, 16, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gemm(NVFP4_W4A4, P, U8(P), F(P), P, F(P), 1 << 20, 64, 128, 1 << 21, P, NVFP4_BF16, 64, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gemm(NVFP4_W4A4, P, U8(P), F(P), P, F(P), huge, huge, 128, 128, P, NVFP4_BF16, huge, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gemm(NVFP4_W4A4, P, U8(P), F(P), P, F(P), 512, 512, 4096, 4096, P, NVFP4_BF16, 512, NULL, 0, NULL) == NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_gemm_requant(NVFP4_W4A4, P, U8(P), F(P), P, F(P), 300, 272, 384, 400, NULL, NVFP4_ACT_NONE, F(P), U8(P),
                            U8(P), NULL, 0, NULL, 0, NULL) == NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_gemm_requant(NVFP4_W4A16, P, NULL, NULL, P, F(P), 64, 40, 128, 128, NULL, NVFP4_ACT_NONE, F(P), U8(P),
                            U8(P), NULL, 0, NULL, 0, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(device_or_hip(nvfp4_gemm(NVFP4_W4A16, P, NULL, NULL, P, F(P), 16, 3072, 12288, 12288, P, NVFP4_BF16, 3072, P,
                                  nvfp4_gemm_workspace_bytes(NVFP4_W4A16, 16, 3072, 12288), NULL)));
  EXPECT(nvfp4_mx_gemm(U8(P), U8(P), U8(P), U8(P), huge, 64, 64, P, NVFP4_BF16, 64, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_mx_quantize(P, NVFP4_BF16, 4, 48, 48, U8(P), U8(P), NULL) == NVFP4_ERR_SHAPE);

  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("abi driver ok\n");
  return failures ? 1 : 0;
}
