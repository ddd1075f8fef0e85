// Device-data precondition scans of the C ABI's debug mode.
//
// The calls document preconditions on the data they read -- finite inputs, tensor scales that are
// finite (and > 0 where the call divides by one), scale bytes that do not encode NaN -- and do not
// check them on the fast path.  With debug checks on, a call first runs these scans over exactly
// the extents it is about to read, waits for them and reports a violation as a status instead of
// computing with the data.  Plain grid-stride loops with one flag word per call: a diagnostic
// pass, not a tuned one.
#include <atomic>

#include "debug_check.hpp"
#include "launch.hpp"

namespace nvfp4 {

// Violation flags, one word per call in flight.  In host code the name is only a stand-in; the
// device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) uint32_t debug_flags[kDebugSlots];

template <int KIND>
__device__ __forceinline__ bool breaks(const uint8_t *row, int64_t c) {
  if constexpr (KIND == kCheckF32) {
    return (reinterpret_cast<const uint32_t *>(row)[c] & 0x7F800000u) == 0x7F800000u;
  } else if constexpr (KIND == kCheckBF16) {
    return (reinterpret_cast<const uint16_t *>(row)[c] & 0x7F80u) == 0x7F80u;
  } else if constexpr (KIND == kCheckE4M3) {
    return (row[c] & 0x7Fu) == 0x7Fu;
  } else {
    return row[c] == 0xFFu;
  }
}

template <int KIND>
__global__ __launch_bounds__(256) void k_debug_scan(const uint8_t *__restrict__ p, int64_t rows, int64_t cols,
                                                    int64_t ld_bytes, uint32_t *flag) {
  const uint64_t n = (uint64_t)rows * (uint64_t)cols;
  bool bad = false;
  for (uint64_t t = blockIdx.x * 256ull + threadIdx.x; t < n; t += (uint64_t)gridDim.x * 256ull) {
    const uint64_t r = t / (uint64_t)cols, c = t % (uint64_t)cols;
    bad |= breaks<KIND>(p + r * (uint64_t)ld_bytes, (int64_t)c);
  }
  if (bad) atomicOr(flag, 1u << KIND);
}

__global__ void k_debug_scale(const float *__restrict__ s, int positive, int kind, uint32_t *flag) {
  if (threadIdx.x == 0) {
    const float v = *s;
    const bool ok = __builtin_isfinite(v) && (!positive || v > 0.0f);
    if (!ok) atomicOr(flag, 1u << kind);
  }
}

static std::atomic<uint32_t *> flags_addr[kMaxDevices];
static std::atomic<unsigned> next_slot{0};

static hipError_t flag_word(uint32_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t *p = flags_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void *q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(debug_flags));
    if (e != hipSuccess) return e;
    if (q == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<uint32_t *>(q);
    flags_addr[dev].store(p, std::memory_order_release);
  }
  *out = p + next_slot.fetch_add(1, std::memory_order_relaxed) % kDebugSlots;
  return hipSuccess;
}

template <int KIND>
static void scan(const DebugRegion &r, uint32_t *flag, hipStream_t stream) {
  const uint64_t n = (uint64_t)r.rows * (uint64_t)r.cols;
  const uint64_t blocks = (n + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  k_debug_scan<KIND><<<grid, 256, 0, stream>>>(static_cast<const uint8_t *>(r.p), r.rows, r.cols, r.ld_bytes, flag);
}

hipError_t debug_scan_regions(const DebugRegion *regions, int n, hipStream_t stream, bool *violated, bool *skipped) {
  *violated = false;
  *skipped = false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) {
    *skipped = true;
    return hipSuccess;
  }
  uint32_t *flag = nullptr;
  e = flag_word(&flag);
  if (e != hipSuccess) return e;
  e = hipMemsetAsync(flag, 0, sizeof(uint32_t), stream);
  if (e != hipSuccess) return e;
  for (int i = 0; i < n; ++i) {
    const DebugRegion &r = regions[i];
    if (r.p == nullptr) continue;
    switch (r.kind) {
      case kCheckScale:
      case kCheckScalePos:
        k_debug_scale<<<1, 64, 0, stream>>>(static_cast<const float *>(r.p), r.kind == kCheckScalePos, r.kind, flag);
        break;
      default:
        if (r.rows <= 0 || r.cols <= 0) break;
        if (r.kind == kCheckF32) scan<kCheckF32>(r, flag, stream);
        else if (r.kind == kCheckBF16) scan<kCheckBF16>(r, flag, stream);
        else if (r.kind == kCheckE4M3) scan<kCheckE4M3>(r, flag, stream);
        else scan<kCheckE8M0>(r, flag, stream);
        break;
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t h = 0;
  e = hipMemcpyAsync(&h, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *violated = h != 0;
  return hipSuccess;
}

}  // namespace nvfp4
