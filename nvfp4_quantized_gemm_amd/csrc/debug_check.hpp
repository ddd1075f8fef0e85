// Device-data precondition scans of the C ABI's debug mode (host declarations).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace nvfp4 {

// What a region must satisfy.  The 2-D kinds scan rows x cols elements at a row pitch of
// ld_bytes; the scalar kinds read one fp32.
enum DebugKind : int {
  kCheckF32 = 0,        // every fp32 finite
  kCheckBF16 = 1,       // every bf16 finite
  kCheckE4M3 = 2,       // no E4M3 scale byte encodes NaN (0x7F, 0xFF)
  kCheckE8M0 = 3,       // no E8M0 scale byte encodes NaN (0xFF)
  kCheckScale = 4,      // a tensor scale that is finite
  kCheckScalePos = 5,   // a tensor scale that is finite and > 0 (the call divides by it)
};

struct DebugRegion {
  const void *p;  // device pointer; NULL or an empty extent skips the region
  int kind;
  int64_t rows, cols, ld_bytes;
};

constexpr int kDebugSlots = 64;  // flag words; calls in flight take them round-robin

// Scan the regions on `stream`, wait for the stream, and set *violated when any region breaks its
// rule.  A stream under graph capture cannot be waited on: then nothing is scanned and *skipped is
// set.  Returns the first HIP error.
hipError_t debug_scan_regions(const DebugRegion *regions, int n, hipStream_t stream, bool *violated, bool *skipped);

}  // namespace nvfp4
