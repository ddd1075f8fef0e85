// libnvfp4 C ABI: argument validation (host only, before any HIP call), device check, dispatch.
// Semantics and layouts are documented in include/nvfp4.h.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "debug_check.hpp"
#include "launch.hpp"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // guards 64-bit size arithmetic

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// M == 0 (an empty tensor) is valid; K must name whole 16-value blocks.
nvfp4_status_t check_mk(int64_t M, int64_t K) {
  if (M < 0 || K < 16 || (K % 16) != 0) return NVFP4_ERR_SHAPE;
  if (M > kMaxElems / K) return NVFP4_ERR_SHAPE;
  if (M * (K / 16) >= ((int64_t)1 << 32)) return NVFP4_ERR_SHAPE;  // 32-bit block index
  return NVFP4_OK;
}

// Block size: values per E4M3 scale byte along K (16, 32 or 64), K a multiple of it.
nvfp4_status_t check_bs(int64_t K, int bs) {
  if (bs != 16 && bs != 32 && bs != 64) return NVFP4_ERR_SHAPE;
  if (K % bs != 0) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

int elem_size(nvfp4_dtype_t t) { return t == NVFP4_F32 ? 4 : 2; }
bool valid_dtype(int t) { return t == NVFP4_F32 || t == NVFP4_BF16; }

// The current device must be gfx950.  Queried once per device index and cached in atomics
// (0 unknown, 1 gfx950, 2 another device), so concurrent callers on any devices are race-free;
// device indices >= kMaxDevices are queried on every call.
nvfp4_status_t check_device() {
  static std::atomic<int8_t> state[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot) {
    const int8_t s = state[dev].load(std::memory_order_acquire);
    if (s != 0) return s == 1 ? NVFP4_OK : NVFP4_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (slot) state[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

// GEMM sizes beyond the 32-bit row / column / depth indices of the kernels.  K and the activation
// pitch are bounded too: the launchers pass K as a 32-bit value and A offsets are formed from lda.
nvfp4_status_t check_gemm_extent(int64_t M, int64_t N, int64_t K, int64_t lda) {
  if (N > kMaxElems / K || M > kMaxElems / N || M >= (1 << 30) || N >= (1 << 30) || K >= (1 << 30))
    return NVFP4_ERR_SHAPE;
  if (lda > kMaxElems / M) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

nvfp4_status_t hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Debug checks: -1 not yet read from NVFP4_DEBUG, 0 off, 1 on.
std::atomic<int> debug_state{-1};

bool debug_on() {
  int d = debug_state.load(std::memory_order_acquire);
  if (d < 0) {
    const char *v = std::getenv("NVFP4_DEBUG");
    int expected = -1;
    debug_state.compare_exchange_strong(expected, (v && v[0] && std::strcmp(v, "0") != 0) ? 1 : 0,
                                        std::memory_order_acq_rel);
    d = debug_state.load(std::memory_order_acquire);
  }
  return d == 1;
}

// With debug checks on, scan the device data a call is about to read (the header lists the rules).
nvfp4_status_t debug_scan(void *stream, std::initializer_list<DebugRegion> regions) {
  if (!debug_on()) return NVFP4_OK;
  bool violated = false, skipped = false;
  if (debug_scan_regions(regions.begin(), (int)regions.size(), static_cast<hipStream_t>(stream), &violated,
                         &skipped) != hipSuccess)
    return NVFP4_ERR_HIP;
  return violated ? NVFP4_ERR_PRECONDITION : NVFP4_OK;
}

// [rows][cols] fp32 or bf16 values at a pitch of ld elements
DebugRegion finite_values(const void *p, nvfp4_dtype_t t, int64_t rows, int64_t cols, int64_t ld) {
  return {p, t == NVFP4_F32 ? kCheckF32 : kCheckBF16, rows, cols, ld * elem_size(t)};
}
// [rows][cols] scale bytes at a pitch of ld bytes
DebugRegion scale_bytes(const void *p, int kind, int64_t rows, int64_t cols, int64_t ld) {
  return {p, kind, rows, cols, ld};
}
DebugRegion tensor_scale_of(const float *s, bool positive) {
  return {s, positive ? kCheckScalePos : kCheckScale, 1, 1, 0};
}
// the scale-byte region of a prepacked [N][K] weight (it follows the code region)
DebugRegion prepacked_scales(const void *b, int64_t N, int64_t K) {
  const int64_t units = ((N + 31) / 32) * ((K + 127) / 128);
  return {static_cast<const uint8_t *>(b) + units * 2048, kCheckE4M3, 1, units * 256, 0};
}

}  // namespace

extern "C" {

const char *nvfp4_status_string(nvfp4_status_t s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (M, N >= 1; K >= 16 and K % 16 == 0)";
    case NVFP4_ERR_STRIDE: return "leading dimension too small";
    case NVFP4_ERR_ALIGN: return "pointer or row pitch misaligned";
    case NVFP4_ERR_DTYPE: return "unsupported dtype";
    case NVFP4_ERR_MODE: return "unknown mode";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    case NVFP4_ERR_DEVICE: return "current device is not gfx950";
    case NVFP4_ERR_PRECONDITION: return "device data breaks a stated precondition (debug checks)";
    default: break;
  }
  return "unknown status";
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

int nvfp4_set_debug_checks(int enable) {
  const int prev = debug_on() ? 1 : 0;
  debug_state.store(enable != 0 ? 1 : 0, std::memory_order_release);
  return prev;
}

size_t nvfp4_quantize_workspace_bytes(int64_t M, int64_t K) {
  (void)M;
  (void)K;
  return (size_t)kAmaxPartials * sizeof(float);
}

}  // extern "C"

namespace {
// Checks shared by the quantize entry points (everything but the workspace).
nvfp4_status_t check_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                              int block_size, const uint8_t *packed, const uint8_t *scales,
                              const float *tensor_scale, nvfp4_scale_mode_t mode, bool *nothing_to_do) {
  *nothing_to_do = false;
  if (!tensor_scale) return NVFP4_ERR_NULL;
  if (!valid_dtype(x_dtype)) return NVFP4_ERR_DTYPE;
  if (mode != NVFP4_SCALE_DYNAMIC && mode != NVFP4_SCALE_STATIC) return NVFP4_ERR_MODE;
  nvfp4_status_t st = check_mk(M, K);
  if (st != NVFP4_OK) return st;
  st = check_bs(K, block_size);
  if (st != NVFP4_OK) return st;
  if (M > 0 && (!x || !packed || !scales)) return NVFP4_ERR_NULL;
  if (M == 0 && mode == NVFP4_SCALE_STATIC) {  // nothing to read or write
    *nothing_to_do = true;
    return NVFP4_OK;
  }
  if (ld_x < K) return NVFP4_ERR_STRIDE;
  const int es = elem_size(x_dtype);
  if (!aligned(x, 16) || ((ld_x * es) % 16) != 0 || !aligned(packed, 8) || !aligned(tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}
}  // namespace

extern "C" {

nvfp4_status_t nvfp4_quantize_bs(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                 int block_size, uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                 nvfp4_scale_mode_t mode, void *workspace, size_t workspace_bytes, void *stream) {
  bool done = false;
  nvfp4_status_t st = check_quantize(x, x_dtype, M, K, ld_x, block_size, packed, scales, tensor_scale, mode, &done);
  if (st != NVFP4_OK || done) return st;
  if (mode == NVFP4_SCALE_DYNAMIC) {
    if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes(M, K)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  }
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {finite_values(x, x_dtype, M, K, ld_x),
                           tensor_scale_of(mode == NVFP4_SCALE_STATIC ? tensor_scale : nullptr, true)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_quantize(x, (int)x_dtype, M, K, ld_x, block_size, packed, scales, tensor_scale,
                                    mode == NVFP4_SCALE_DYNAMIC, static_cast<float *>(workspace),
                                    static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_quantize_noalloc(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                      int block_size, uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                      nvfp4_scale_mode_t mode, void *stream) {
  bool done = false;
  nvfp4_status_t st = check_quantize(x, x_dtype, M, K, ld_x, block_size, packed, scales, tensor_scale, mode, &done);
  if (st != NVFP4_OK || done) return st;
  // the library's scratch must hold what the call needs (the dynamic pass's partial maxima)
  if (mode == NVFP4_SCALE_DYNAMIC && nvfp4_quantize_workspace_bytes(M, K) > kQuantizeScratchBytes)
    return NVFP4_ERR_WORKSPACE;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {finite_values(x, x_dtype, M, K, ld_x),
                           tensor_scale_of(mode == NVFP4_SCALE_STATIC ? tensor_scale : nullptr, true)});
  if (st != NVFP4_OK) return st;
  float *partial = nullptr;
  if (mode == NVFP4_SCALE_DYNAMIC) {
    st = hip_status(quantize_scratch(&partial));
    if (st != NVFP4_OK) return st;
  }
  return hip_status(launch_quantize(x, (int)x_dtype, M, K, ld_x, block_size, packed, scales, tensor_scale,
                                    mode == NVFP4_SCALE_DYNAMIC, partial, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                              uint8_t *packed, uint8_t *scales, float *tensor_scale, nvfp4_scale_mode_t mode,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return nvfp4_quantize_bs(x, x_dtype, M, K, ld_x, 16, packed, scales, tensor_scale, mode, workspace, workspace_bytes,
                           stream);
}

nvfp4_status_t nvfp4_fake_quantize_bs(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                      int block_size, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                      float *tensor_scale, nvfp4_scale_mode_t mode, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!tensor_scale) return NVFP4_ERR_NULL;
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return NVFP4_ERR_DTYPE;
  if (mode != NVFP4_SCALE_DYNAMIC && mode != NVFP4_SCALE_STATIC) return NVFP4_ERR_MODE;
  nvfp4_status_t st = check_mk(M, K);
  if (st != NVFP4_OK) return st;
  st = check_bs(K, block_size);
  if (st != NVFP4_OK) return st;
  if (M > 0 && (!x || !y)) return NVFP4_ERR_NULL;
  if (M == 0 && mode == NVFP4_SCALE_STATIC) return NVFP4_OK;  // nothing to read or write
  if (ld_x < K || ld_y < K) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || ((ld_x * elem_size(x_dtype)) % 16) != 0 || !aligned(y, 16) ||
      ((ld_y * elem_size(y_dtype)) % 16) != 0 || !aligned(tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  if (mode == NVFP4_SCALE_DYNAMIC) {
    if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes(M, K)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  }
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {finite_values(x, x_dtype, M, K, ld_x),
                           tensor_scale_of(mode == NVFP4_SCALE_STATIC ? tensor_scale : nullptr, true)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_fake_quantize(x, (int)x_dtype, M, K, ld_x, block_size, y, (int)y_dtype, ld_y,
                                         tensor_scale, mode == NVFP4_SCALE_DYNAMIC, static_cast<float *>(workspace),
                                         static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_fake_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                   void *y, nvfp4_dtype_t y_dtype, int64_t ld_y, float *tensor_scale,
                                   nvfp4_scale_mode_t mode, void *workspace, size_t workspace_bytes, void *stream) {
  return nvfp4_fake_quantize_bs(x, x_dtype, M, K, ld_x, 16, y, y_dtype, ld_y, tensor_scale, mode, workspace,
                                workspace_bytes, stream);
}

nvfp4_status_t nvfp4_dequantize_bs(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                   int64_t M, int64_t K, int block_size, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                   void *stream) {
  if (!valid_dtype(y_dtype)) return NVFP4_ERR_DTYPE;
  nvfp4_status_t st = check_mk(M, K);
  if (st != NVFP4_OK) return st;
  st = check_bs(K, block_size);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;  // empty: nothing to read or write
  if (!packed || !scales || !tensor_scale || !y) return NVFP4_ERR_NULL;
  if (ld_y < K) return NVFP4_ERR_STRIDE;
  const int es = elem_size(y_dtype);
  if (!aligned(y, 16) || ((ld_y * es) % 16) != 0 || !aligned(packed, 8) || !aligned(tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {scale_bytes(scales, kCheckE4M3, M, K / block_size, K / block_size),
                           tensor_scale_of(tensor_scale, false)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_dequantize(packed, scales, tensor_scale, M, K, block_size, y, (int)y_dtype, ld_y,
                                      static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t M,
                                int64_t K, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y, void *stream) {
  return nvfp4_dequantize_bs(packed, scales, tensor_scale, M, K, 16, y, y_dtype, ld_y, stream);
}

size_t nvfp4_prepacked_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 16 || (K % 16) != 0 || N > kMaxElems / K) return 0;
  const int64_t Nu = (N + 31) / 32, Kc = (K + 127) / 128;
  return (size_t)(Nu * Kc * (2048 + 256));
}

nvfp4_status_t nvfp4_prepack_weight_bs(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K,
                                       int block_size, void *prepacked, void *stream) {
  nvfp4_status_t st = check_mk(N, K);
  if (st != NVFP4_OK) return st;
  st = check_bs(K, block_size);
  if (st != NVFP4_OK) return st;
  if (N == 0) return NVFP4_OK;  // empty weight
  if (!packed || !scales || !prepacked) return NVFP4_ERR_NULL;
  if (!aligned(prepacked, 16)) return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {scale_bytes(scales, kCheckE4M3, N, K / block_size, K / block_size)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_prepack(packed, scales, N, K, block_size, prepacked, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_prepack_weight(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K,
                                    void *prepacked, void *stream) {
  return nvfp4_prepack_weight_bs(packed, scales, N, K, 16, prepacked, stream);
}

nvfp4_status_t nvfp4_unpack_weight_bs(const void *prepacked, int64_t N, int64_t K, int block_size, uint8_t *packed,
                                      uint8_t *scales, void *stream) {
  nvfp4_status_t st = check_mk(N, K);
  if (st != NVFP4_OK) return st;
  st = check_bs(K, block_size);
  if (st != NVFP4_OK) return st;
  if (N == 0) return NVFP4_OK;  // empty weight
  if (!packed || !scales || !prepacked) return NVFP4_ERR_NULL;
  if (!aligned(prepacked, 16)) return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  return hip_status(launch_unpack(prepacked, N, K, block_size, packed, scales, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_unpack_weight(const void *prepacked, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales,
                                   void *stream) {
  return nvfp4_unpack_weight_bs(prepacked, N, K, 16, packed, scales, stream);
}

size_t nvfp4_gemm_workspace_bytes_ld(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  if (mode != NVFP4_W4A4 && mode != NVFP4_W4A16) return 0;
  if (M < 1 || N < 1 || K < 16 || (K % 16) != 0 || lda < K) return 0;  // empty or invalid calls
  if (check_gemm_extent(M, N, K, lda) != NVFP4_OK) return 0;
  return gemm_workspace_bytes((int)mode, M, N, K, lda);
}

size_t nvfp4_gemm_workspace_bytes(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K) {
  return nvfp4_gemm_workspace_bytes_ld(mode, M, N, K, K);
}

nvfp4_status_t nvfp4_gemm_bs(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                             const float *a_tensor_scale, int a_block_size, const void *b_prepacked,
                             const float *b_tensor_scale, int64_t M, int64_t N, int64_t K, int64_t lda, void *c,
                             nvfp4_dtype_t c_dtype, int64_t ldc, void *workspace, size_t workspace_bytes,
                             void *stream) {
  if (mode != NVFP4_W4A4 && mode != NVFP4_W4A16) return NVFP4_ERR_MODE;
  if (mode == NVFP4_W4A4 && check_bs(K, a_block_size) != NVFP4_OK) return NVFP4_ERR_SHAPE;
  if (mode == NVFP4_W4A16 && (a_scales || a_tensor_scale)) return NVFP4_ERR_NULL;
  if (!valid_dtype(c_dtype)) return NVFP4_ERR_DTYPE;
  if (N < 0) return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_mk(M, K);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;  // empty output: nothing to read or write
  if (!a || !b_prepacked || !b_tensor_scale || !c) return NVFP4_ERR_NULL;
  if (mode == NVFP4_W4A4 && (!a_scales || !a_tensor_scale)) return NVFP4_ERR_NULL;
  if (lda < K || ldc < N) return NVFP4_ERR_STRIDE;
  st = check_gemm_extent(M, N, K, lda);
  if (st != NVFP4_OK) return st;
  if (mode == NVFP4_W4A4) {
    if ((lda % a_block_size) != 0) return NVFP4_ERR_STRIDE;  // whole scale blocks per row
    if (!aligned(a, 8) || !aligned(a_scales, 4)) return NVFP4_ERR_ALIGN;
  } else {
    if (!aligned(a, 16) || ((lda * 2) % 16) != 0) return NVFP4_ERR_ALIGN;
  }
  if (!aligned(b_prepacked, 16) || !aligned(c, 16) || !aligned(b_tensor_scale, 4)) return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_gemm_workspace_bytes_ld(mode, M, N, K, lda);  // the plan the launch runs
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  }
  st = check_device();
  if (st != NVFP4_OK) return st;
  if (mode == NVFP4_W4A4)
    st = debug_scan(stream, {scale_bytes(a_scales, kCheckE4M3, M, K / a_block_size, lda / a_block_size),
                             tensor_scale_of(a_tensor_scale, false), prepacked_scales(b_prepacked, N, K),
                             tensor_scale_of(b_tensor_scale, false)});
  else
    st = debug_scan(stream, {finite_values(a, NVFP4_BF16, M, K, lda), prepacked_scales(b_prepacked, N, K),
                             tensor_scale_of(b_tensor_scale, false)});
  if (st != NVFP4_OK) return st;
  GemmArgs g;
  g.mode = (int)mode;
  g.a = a;
  g.a_scales = a_scales;
  g.a_ts = a_tensor_scale;
  g.b = b_prepacked;
  g.b_ts = b_tensor_scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.a_blk = (mode == NVFP4_W4A4) ? a_block_size : 16;
  g.c = c;
  g.out_dtype = (int)c_dtype;
  g.ldc = ldc;
  g.workspace = workspace;
  return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales, const float *a_tensor_scale,
                          const void *b_prepacked, const float *b_tensor_scale, int64_t M, int64_t N, int64_t K,
                          int64_t lda, void *c, nvfp4_dtype_t c_dtype, int64_t ldc, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return nvfp4_gemm_bs(mode, a, a_scales, a_tensor_scale, 16, b_prepacked, b_tensor_scale, M, N, K, lda, c, c_dtype,
                       ldc, workspace, workspace_bytes, stream);
}

// ---- GEMM with NVFP4 output ------------------------------------------------------------------

size_t nvfp4_gemm_requant_workspace_bytes_ld(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  if (mode != NVFP4_W4A4 && mode != NVFP4_W4A16) return 0;
  if (M < 1 || N < 1 || K < 16 || (K % 16) != 0 || (N % 16) != 0 || lda < K) return 0;  // empty or invalid
  if (check_gemm_extent(M, N, K, lda) != NVFP4_OK) return 0;
  return gemm_requant_workspace_bytes((int)mode, M, N, K, lda);
}

size_t nvfp4_gemm_requant_workspace_bytes(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K) {
  return nvfp4_gemm_requant_workspace_bytes_ld(mode, M, N, K, K);
}

nvfp4_status_t nvfp4_gemm_requant_bs(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                                     const float *a_tensor_scale, int a_block_size, const void *b_prepacked,
                                     const float *b_tensor_scale, int64_t M, int64_t N, int64_t K, int64_t lda,
                                     const float *bias, nvfp4_act_t act, const float *out_tensor_scale,
                                     uint8_t *out_packed, uint8_t *out_scales, float *y, int64_t ld_y, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (mode != NVFP4_W4A4 && mode != NVFP4_W4A16) return NVFP4_ERR_MODE;
  if (mode == NVFP4_W4A4 && check_bs(K, a_block_size) != NVFP4_OK) return NVFP4_ERR_SHAPE;
  if (mode == NVFP4_W4A16 && (a_scales || a_tensor_scale)) return NVFP4_ERR_NULL;
  if (act != NVFP4_ACT_NONE && act != NVFP4_ACT_GELU_TANH) return NVFP4_ERR_MODE;
  if (N < 0 || (N % 16) != 0) return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_mk(M, K);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;  // empty output: nothing to read or write
  if (!a || !b_prepacked || !b_tensor_scale || !out_tensor_scale || !out_packed || !out_scales)
    return NVFP4_ERR_NULL;
  if (mode == NVFP4_W4A4 && (!a_scales || !a_tensor_scale)) return NVFP4_ERR_NULL;
  if (lda < K) return NVFP4_ERR_STRIDE;
  st = check_gemm_extent(M, N, K, lda);
  if (st != NVFP4_OK) return st;
  if (y && (ld_y < N || (ld_y % 4) != 0)) return NVFP4_ERR_STRIDE;
  if (mode == NVFP4_W4A4) {
    if ((lda % a_block_size) != 0) return NVFP4_ERR_STRIDE;  // whole scale blocks per row
    if (!aligned(a, 8) || !aligned(a_scales, 4)) return NVFP4_ERR_ALIGN;
  } else {
    if (!aligned(a, 16) || ((lda * 2) % 16) != 0) return NVFP4_ERR_ALIGN;
  }
  if (!aligned(b_prepacked, 16) || !aligned(b_tensor_scale, 4) || !aligned(out_tensor_scale, 4) ||
      !aligned(out_packed, 16) || (bias && !aligned(bias, 16)) || (y && !aligned(y, 16)))
    return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_gemm_requant_workspace_bytes_ld(mode, M, N, K, lda);  // the plan the launch runs
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  }
  st = check_device();
  if (st != NVFP4_OK) return st;
  if (mode == NVFP4_W4A4)
    st = debug_scan(stream, {scale_bytes(a_scales, kCheckE4M3, M, K / a_block_size, lda / a_block_size),
                             tensor_scale_of(a_tensor_scale, false), prepacked_scales(b_prepacked, N, K),
                             tensor_scale_of(b_tensor_scale, false), finite_values(bias, NVFP4_F32, 1, N, N),
                             tensor_scale_of(out_tensor_scale, true)});
  else
    st = debug_scan(stream, {finite_values(a, NVFP4_BF16, M, K, lda), prepacked_scales(b_prepacked, N, K),
                             tensor_scale_of(b_tensor_scale, false), finite_values(bias, NVFP4_F32, 1, N, N),
                             tensor_scale_of(out_tensor_scale, true)});
  if (st != NVFP4_OK) return st;
  GemmArgs g;
  g.mode = (int)mode;
  g.a = a;
  g.a_scales = a_scales;
  g.a_ts = a_tensor_scale;
  g.b = b_prepacked;
  g.b_ts = b_tensor_scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.c = nullptr;
  g.out_dtype = 2;
  g.ldc = 0;
  g.workspace = workspace;
  g.qo.bias = bias;
  g.qo.out_ts = out_tensor_scale;
  g.qo.packed = out_packed;
  g.qo.scales = out_scales;
  g.qo.y = y;
  g.qo.ldy = ld_y;
  g.qo.act = (int)act;
  g.a_blk = (mode == NVFP4_W4A4) ? a_block_size : 16;
  return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_gemm_requant(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                                  const float *a_tensor_scale, const void *b_prepacked, const float *b_tensor_scale,
                                  int64_t M, int64_t N, int64_t K, int64_t lda, const float *bias, nvfp4_act_t act,
                                  const float *out_tensor_scale, uint8_t *out_packed, uint8_t *out_scales, float *y,
                                  int64_t ld_y, void *workspace, size_t workspace_bytes, void *stream) {
  return nvfp4_gemm_requant_bs(mode, a, a_scales, a_tensor_scale, 16, b_prepacked, b_tensor_scale, M, N, K, lda, bias,
                               act, out_tensor_scale, out_packed, out_scales, y, ld_y, workspace, workspace_bytes,
                               stream);
}

// ---- MXFP4 ------------------------------------------------------------------------------------

namespace {
nvfp4_status_t check_mx_mk(int64_t M, int64_t K) {
  if (M < 0 || K < 32 || (K % 32) != 0) return NVFP4_ERR_SHAPE;
  if (M > kMaxElems / K) return NVFP4_ERR_SHAPE;
  if (M * (K / 16) >= ((int64_t)1 << 32)) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}
}  // namespace

nvfp4_status_t nvfp4_mx_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                 uint8_t *packed, uint8_t *scales, void *stream) {
  if (!valid_dtype(x_dtype)) return NVFP4_ERR_DTYPE;
  nvfp4_status_t st = check_mx_mk(M, K);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;
  if (!x || !packed || !scales) return NVFP4_ERR_NULL;
  if (ld_x < K) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || ((ld_x * elem_size(x_dtype)) % 16) != 0 || !aligned(packed, 8)) return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {finite_values(x, x_dtype, M, K, ld_x)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_mx_quantize(x, (int)x_dtype, M, K, ld_x, packed, scales, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, void *y,
                                   nvfp4_dtype_t y_dtype, int64_t ld_y, void *stream) {
  if (!valid_dtype(y_dtype)) return NVFP4_ERR_DTYPE;
  nvfp4_status_t st = check_mx_mk(M, K);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;
  if (!packed || !scales || !y) return NVFP4_ERR_NULL;
  if (ld_y < K) return NVFP4_ERR_STRIDE;
  if (!aligned(y, 16) || ((ld_y * elem_size(y_dtype)) % 16) != 0 || !aligned(packed, 8)) return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {scale_bytes(scales, kCheckE8M0, M, K / 32, K / 32)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_mx_dequantize(packed, scales, M, K, y, (int)y_dtype, ld_y, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_mx_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b, const uint8_t *b_scales,
                             int64_t M, int64_t N, int64_t K, void *c, nvfp4_dtype_t c_dtype, int64_t ldc,
                             void *stream) {
  if (!valid_dtype(c_dtype)) return NVFP4_ERR_DTYPE;
  if (N < 0) return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_mx_mk(M, K);
  if (st != NVFP4_OK) return st;
  st = check_mx_mk(N, K);
  if (st != NVFP4_OK) return st;
  if (M >= (1 << 30) || N >= (1 << 30) || (N > 0 && M > kMaxElems / N)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a || !a_scales || !b || !b_scales || !c) return NVFP4_ERR_NULL;
  if (ldc < N) return NVFP4_ERR_STRIDE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) || !aligned(c, 16))
    return NVFP4_ERR_ALIGN;
  st = check_device();
  if (st != NVFP4_OK) return st;
  st = debug_scan(stream, {scale_bytes(a_scales, kCheckE8M0, M, K / 32, K / 32),
                           scale_bytes(b_scales, kCheckE8M0, N, K / 32, K / 32)});
  if (st != NVFP4_OK) return st;
  return hip_status(launch_mx_gemm(a, a_scales, b, b_scales, M, N, K, c, (int)c_dtype, ldc,
                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"
