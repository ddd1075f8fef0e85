// Output epilogue shared by the tiled GEMM kernels (gfx950).
#pragma once
#include "common.hpp"

namespace nvfp4 {

// Output staging.  The MFMAs compute C^T tiles (the B fragment is the row operand), so lane l of
// 32x32 tile (i, j) holds output row r = l % 32 of the tile and, for g = 0..3, the four consecutive
// columns 8 g + 4 (l / 32) + 0..3.  Each 32-row slab of a wave's sub-tile is written to a
// wave-private, padded, row-major LDS region (one 8- or 16-byte write per column group) and read
// back row-contiguously, so every global store instruction covers whole rows of the sub-tile with
// 16-byte lane stores.  `vec` says the rows of C are 16-byte aligned; a lane whose 16 bytes lie
// inside C stores them at once, lanes at the ragged edge store element by element.
template <int CW, int ES>
struct EpiPitch {
  static constexpr int kPitch = CW * ES + 16;  // row pitch in bytes (16-B pad against bank conflicts)
};

__device__ __forceinline__ void wave_lds_sync() {
  // LDS accesses of one wave complete in order; this only keeps the compiler from reordering them.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int CW, int TM, int TN, typename OutT>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TM][TN], float scale, OutT *__restrict__ C,
                                           int64_t ldc, int M, int N, int row0, int col0, bool vec,
                                           uint8_t *lds, int lane) {
  constexpr int ES = (int)sizeof(OutT);
  constexpr int kPitch = EpiPitch<CW, ES>::kPitch;
  constexpr int kLanesPerRow = CW * ES / 16;
  constexpr int kRowsPerRead = 64 / kLanesPerRow;
  constexpr int kEl = 16 / ES;  // elements per 16-byte lane access
  static_assert(CW == 32 * TN && kLanesPerRow <= 64 && 64 % kLanesPerRow == 0, "epilogue shape");
  const int lr = lane & 31, lh = lane >> 5;
  const int rr = lane / kLanesPerRow, cq = (lane % kLanesPerRow) * kEl;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v0 = acc[i][j][4 * g] * scale, v1 = acc[i][j][4 * g + 1] * scale;
        const float v2 = acc[i][j][4 * g + 2] * scale, v3 = acc[i][j][4 * g + 3] * scale;
        uint8_t *p = lds + lr * kPitch + (j * 32 + 8 * g + 4 * lh) * ES;
        if (ES == 4) {
          const u32x4 o = {__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
          *reinterpret_cast<u32x4 *>(p) = o;
        } else {
          const bf16x2 h0 = {(__bf16)v0, (__bf16)v1}, h1 = {(__bf16)v2, (__bf16)v3};
          const u32x2 o = {__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
          *reinterpret_cast<u32x2 *>(p) = o;
        }
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 32 / kRowsPerRead; ++t) {
      const int r = t * kRowsPerRead + rr;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + r * kPitch + cq * ES);
      const int row = row0 + i * 32 + r, col = col0 + cq;
      OutT *pc = C + (int64_t)row * ldc + col;
      if (vec && row < M && col + kEl <= N) {
        *reinterpret_cast<u32x4 *>(pc) = v;
      } else if (row < M && col < N) {
        // ragged edge: element by element (elements taken out of the registers by shifts, so the
        // staged vector never goes through memory)
#pragma unroll
        for (int q = 0; q < kEl; ++q) {
          if (col + q < N) {
            const uint32_t word = v[(q * ES) / 4];
            if (ES == 4) reinterpret_cast<uint32_t *>(pc)[q] = word;
            else reinterpret_cast<uint16_t *>(pc)[q] = (uint16_t)(word >> (16 * (q & 1)));
          }
        }
      }
    }
    wave_lds_sync();  // the next slab overwrites this region
  }
}

}  // namespace nvfp4
