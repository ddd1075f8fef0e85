// Internal interface between the C ABI (nvfp4_api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// Per-device, per-kernel one-time setup of the dynamic LDS limit (kernels whose LDS exceeds the
// default).  `done` is one flag array per kernel instantiation.  Thread-safe: concurrent first
// calls on a device may both set the attribute, which is idempotent; a flag is only raised after
// a successful call.  Devices with an index >= kMaxDevices set it on every launch.
constexpr int kMaxDevices = 64;
inline hipError_t set_dynamic_lds(const void *kern, int bytes, std::atomic<bool> *done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && slot) done[dev].store(true, std::memory_order_release);
  return e;
}

constexpr int kAmaxPartials = 1024;     // max workgroups of the dynamic amax pass (= partials)
// Grid caps (grid-stride beyond).  The quantize kernel runs at most 1280 workgroups, the five per
// CU that its 96 registers allow at once, each prefetching its next tile (2048, which left a
// second partial round, was 0.5-0.8 us slower on 37.7 and 63 MB activations); tensors with more
// than 8192 workgroups' worth of tiles run 16384 (measured faster for every pass there).  The
// MXFP4 quantize keeps 2048.  The dequantize kernel, write-dominated, runs one workgroup per four
// tiles up to a large cap.
constexpr int kQuantizeMaxGrid = 1280;
constexpr int kQuantizeWideFrom = 8192;
constexpr int kQuantizeWideGrid = 16384;
constexpr int kMxQuantizeMaxGrid = 2048;
constexpr int kDequantizeMaxGrid = 1 << 20;

// blk: values per E4M3 scale byte along K (16, 32 or 64)
hipError_t launch_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, int blk, uint8_t *packed,
                           uint8_t *scales, float *tensor_scale, bool dynamic, float *partial, hipStream_t stream);
// Library-owned device scratch for the dynamic pass's partial maxima (the no-allocation entry
// point): kQuantizeScratchBytes per GPU; *ptr receives the current device's address of it.
constexpr size_t kQuantizeScratchBytes = (size_t)kAmaxPartials * sizeof(float);
hipError_t quantize_scratch(float **ptr);
// Fake quantization: y = dequantize(quantize(x)) in one pass (no NVFP4 tensor is written).
hipError_t launch_fake_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, int blk, void *y,
                                int y_dtype, int64_t ld_y, float *tensor_scale, bool dynamic, float *partial,
                                hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t M,
                             int64_t K, int blk, void *y, int out_dtype, int64_t ld_y, hipStream_t stream);

hipError_t launch_prepack(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K, int blk, void *out,
                          hipStream_t stream);
hipError_t launch_unpack(const void *in, int64_t N, int64_t K, int blk, uint8_t *packed, uint8_t *scales,
                         hipStream_t stream);

// W4A16_128x256h: 128 x 256 tiles with half-chunk stages, two workgroups per CU; W4A16_64x256: 64-row tiles
enum class GemmVariant {
  Generic, W4A4_256x256, W4A4_128x128, W4A4_128x192, W4A16_128x256, W4A16_128x256h, W4A16_64x256, W4A16_Skinny
};

struct GemmPlan {
  GemmVariant variant = GemmVariant::Generic;
  int splits = 1;     // K splits (partial tiles reduced by a second kernel)
  int waves = 4;      // W4A16_Skinny: waves per workgroup
  int64_t n_big = 0;  // > 0: columns [0, n_big) in 256x256 tiles, the rest in 128x128 tiles
};

// NVFP4 output of the GEMM (epilogue-fused requantization): y = acc S_A S_B (+ bias) (-> act),
// quantized under the static tensor scale *out_ts into canonical packed [M][N/2] / scales [M][N/16];
// optionally also written as fp32 to y [M][ldy].
constexpr int kActNone = 0, kActGeluTanh = 1;
struct QuantOut {
  const float *bias = nullptr;    // [N] fp32 or null
  const float *out_ts = nullptr;  // device fp32 static tensor scale of the output
  uint8_t *packed = nullptr;
  uint8_t *scales = nullptr;
  float *y = nullptr;
  int64_t ldy = 0;
  int act = kActNone;
};

struct GemmArgs {
  int mode;  // 0 W4A4, 1 W4A16
  const void *a;
  const uint8_t *a_scales;
  int a_blk = 16;  // W4A4: values per A scale byte along K (16, 32 or 64)
  const float *a_ts;
  const void *b;
  const float *b_ts;
  int64_t M, N, K, lda;
  void *c;
  int out_dtype;  // 0 f32, 1 bf16, 2 NVFP4 (qo)
  int64_t ldc;
  void *workspace;
  QuantOut qo;
};

GemmPlan plan_gemm(int mode, int64_t M, int64_t N, int64_t K, int64_t lda);
// Workspace of exactly the plan launch_gemm runs for these arguments (the activation's row pitch
// lda decides between the tiled and the generic kernels, so it is part of the plan).
size_t gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K, int64_t lda);
// workspace of the NVFP4-output GEMM: fp32 partials wherever the plan does not end in a tile kernel
size_t gemm_requant_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K, int64_t lda);
hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream);

// W4A16 with M <= kSkinnyMaxM: streaming kernel over the prepacked weight (gemm_skinny.hip)
constexpr int kSkinnyMaxM = 64;
hipError_t launch_gemm_skinny(const GemmArgs &g, int waves, int splits, float *partial, hipStream_t stream);

// C = (sum of the splits' fp32 partials [splits][M][N], in order) * (a_ts ? *a_ts : 1) *
// (b_ts ? *b_ts : 1); needs N % 4 == 0 (N % 16 == 0 for out_dtype 2, which writes qo)
hipError_t launch_splitk_reduce(const float *partial, int splits, int64_t M, int64_t N, void *c, int out_dtype,
                                int64_t ldc, const float *a_ts, const float *b_ts, const QuantOut &qo,
                                hipStream_t stream);

// MXFP4 (mxfp4.hip): 32-value blocks with E8M0 scales, GEMM on the block-scaled FP4 MFMA.
hipError_t launch_mx_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, uint8_t *packed,
                              uint8_t *scales, hipStream_t stream);
hipError_t launch_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, void *y,
                                int out_dtype, int64_t ld_y, hipStream_t stream);
hipError_t launch_mx_gemm(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int64_t M,
                          int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc, hipStream_t stream);

}  // namespace nvfp4
