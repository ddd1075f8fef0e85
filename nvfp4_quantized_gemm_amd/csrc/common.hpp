// Device helpers shared by the libnvfp4 kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Largest finite E4M3FN magnitude and the dynamic-scale divisor 6 * 448.
constexpr float kE4M3Max = 448.0f;
constexpr float kDynDivisor = 2688.0f;

// Fast-path validity window for the tensor scale: inside it every reciprocal used by the
// quantizer's fast path is a normal fp32 value.
constexpr float kFastSMin = 0x1p-100f;
constexpr float kFastSMax = 0x1p+100f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// OCP E4M3FN byte -> fp32 (hardware conversion; gfx950 decodes the OCP variant).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Hardware FP4 conversions; the byte-select operand must be a literal, hence the templates.
// Encode: two fp32 -> two E2M1 codes (round-half-even, saturating at +-6, sign kept) into byte J.
template <int J>
__device__ __forceinline__ uint32_t fp4_encode2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, J);
}
// Decode byte J of `codes` (low nibble first) to exact values.
template <int J>
__device__ __forceinline__ f32x2 fp4_decode2_f32(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, J);
}
template <int J>
__device__ __forceinline__ f16x2 fp4_decode2_f16(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, J);
}

// Magic-number unsigned division by a runtime constant d (1 <= d < 2^31).
struct FastDiv {
  uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.mul = (uint32_t)((((1ull << 32) * ((1ull << s) - d)) / d) + 1);
  return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv &f) {
  if (f.shift == 0) return n;  // d == 1
  uint32_t t = __umulhi(n, f.mul);
  return (t + ((n - t) >> 1)) >> (f.shift - 1);
}

// Lane swaps within quads of lanes (DPP quad_perm): lane i reads lane i ^ 1, or lane i ^ 2.
__device__ __forceinline__ float swap_lane1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap_lane2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copies (gfx950 LDS-DMA): every lane supplies its own global address; the
// wave's data lands contiguously at `lds` (lane i at lds + i * size).  `lds` must be wave-uniform.
__device__ __forceinline__ void g2l16(const void *g, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2l4(const void *g, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 4, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are outstanding (they complete in
// issue order), then meet the other waves at a bare barrier: unlike __syncthreads() this does not
// also wait for the loads issued after the ones needed.
template <int N>
__device__ __forceinline__ void wait_vmem_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Grouped raster over a tiles_m x tiles_n tile grid (bijective): consecutive indices walk down
// groups of G tile rows before moving right, so a run of consecutive tiles (one XCD's share of a
// round) touches about G row blocks of A and run / G column blocks of B instead of one row and
// the whole width.
template <int G>
__device__ __forceinline__ void grouped_tile(int j, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int group_size = G * tiles_n;
  const int group = j / group_size, r = j - group * group_size;
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  tm = first_m + r % gm;
  tn = r / gm;
}

// Lane swaps across quads: lane i reads lane i ^ 4, or lane i ^ 8 (ds_swizzle bit mode, xor masks).
__device__ __forceinline__ float swap_lane4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}
__device__ __forceinline__ float swap_lane8(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
}

// Maximum over the LPB adjacent lanes of an aligned group (LPB = 1, 2, 4, 8 or 16).
template <int LPB>
__device__ __forceinline__ float group_max(float v) {
  if (LPB >= 2) v = fmaxf(v, swap_lane1(v));
  if (LPB >= 4) v = fmaxf(v, swap_lane2(v));
  if (LPB >= 8) v = fmaxf(v, swap_lane4(v));
  if (LPB >= 16) v = fmaxf(v, swap_lane8(v));
  return v;
}

// Lane-contiguous element mapping of the bandwidth kernels.  A tensor of M rows x K (K a multiple
// of the block size BLK) is cut into segments of EPL consecutive elements along K, numbered
// row-major; EPL is chosen so that a segment is 16 bytes of the wide side (8 bf16 or 4 fp32), and
// consecutive lanes take consecutive segments, so every wave-wide load or store covers one
// contiguous span.  Segment g lies in block g / LPB (LPB = BLK / EPL adjacent lanes share a block).
template <int EPL, int BLK = 16>
struct Segments {
  static constexpr int kLanesPerBlock = BLK / EPL;
  static constexpr int kShift = (kLanesPerBlock == 2) ? 1 : (kLanesPerBlock == 4) ? 2 : (kLanesPerBlock == 8) ? 3 : 4;
  static_assert(EPL == 8 || EPL == 4, "segments are 8 or 4 elements");
  static_assert(kLanesPerBlock == 2 || kLanesPerBlock == 4 || kLanesPerBlock == 8 || kLanesPerBlock == 16,
                "lanes per block");
  // element offset of segment g in a tensor with row stride ld (elements); rows of exactly K
  // elements (DENSE) need no division, otherwise bpr divides by the blocks per row
  template <bool DENSE>
  __device__ static uint64_t offset(uint64_t g, const FastDiv &bpr, int64_t ld) {
    if (DENSE) return g * EPL;
    const uint32_t blk = (uint32_t)(g >> kShift);
    const uint32_t row = fastdiv(blk, bpr);
    const uint32_t col = (blk - row * bpr.d) * BLK + (uint32_t)(g & (kLanesPerBlock - 1)) * EPL;
    return (uint64_t)row * (uint64_t)ld + col;
  }
};

// Input loading of the bandwidth kernels: one 16-byte segment per lane (raw), then unpacked to fp32.

template <int DT>
struct SegIn;

// NT: a streaming (non-temporal) load, for data that is read once: it keeps the caches for data
// that is reused and streams markedly faster from HBM.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const void *p) {
  const u32x4 *q = static_cast<const u32x4 *>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

template <bool NT>
__device__ __forceinline__ void store16(void *p, const u32x4 &v) {
  u32x4 *q = static_cast<u32x4 *>(p);
  if constexpr (NT) __builtin_nontemporal_store(v, q);
  else *q = v;
}

template <>
struct SegIn<0> {  // fp32: 4 values
  static constexpr int kElems = 4;
  template <bool NT = false>
  __device__ static u32x4 raw(const void *base, uint64_t elem_off) {
    return load16<NT>(static_cast<const float *>(base) + elem_off);
  }
  __device__ static void unpack(const u32x4 &w, float v[4]) {
    v[0] = __uint_as_float(w.x);
    v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z);
    v[3] = __uint_as_float(w.w);
  }
};

template <>
struct SegIn<1> {  // bf16: 8 values
  static constexpr int kElems = 8;
  template <bool NT = false>
  __device__ static u32x4 raw(const void *base, uint64_t elem_off) {
    return load16<NT>(static_cast<const uint16_t *>(base) + elem_off);
  }
  __device__ static void unpack(const u32x4 &w, float v[8]) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = bf16lo(a[t]);
      v[2 * t + 1] = bf16hi(a[t]);
    }
  }
};

}  // namespace nvfp4
