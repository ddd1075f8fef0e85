// Output epilogue shared by the tiled GEMM kernels (gfx950).
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "quant_core.hpp"

namespace nvfp4 {

// Output staging.  The MFMAs compute C^T tiles (the B fragment is the row operand), so lane l of
// 32x32 tile (i, j) holds output row r = l % 32 of the tile and, for g = 0..3, the four consecutive
// columns 8 g + 4 (l / 32) + 0..3.  Each 32-row slab of a wave's sub-tile is written to a
// wave-private, padded, row-major LDS region (one 8- or 16-byte write per column group) and read
// back row-contiguously, so every global store instruction covers whole rows of the sub-tile with
// 16-byte lane stores.  `vec` says the rows of C are 16-byte aligned; a lane whose 16 bytes lie
// inside C stores them at once, lanes at the ragged edge store element by element.  A sub-tile
// width that is not a power of two (96 columns) is read back as two pieces (64 + 32 columns), each
// with a whole number of rows per 64-lane read.
template <int CW, int ES>
struct EpiPitch {
  static constexpr int kPitch = CW * ES + 16;  // row pitch in bytes (16-B pad against bank conflicts)
};

// The first read-back piece of a CW-column slab: the largest power of two <= CW (at most 128);
// the rest (CW minus that) must itself be 0 or a power of two.
template <int CW>
struct EpiPieces {
  static constexpr int kFirst = CW >= 128 ? 128 : (CW >= 64 ? 64 : 32);
  static constexpr int kRest = CW - kFirst;
  static_assert(CW % 32 == 0 && CW <= 256, "epilogue width");
  static_assert(kRest == 0 || kRest == 32 || kRest == 64 || kRest == 128, "epilogue pieces");
};

__device__ __forceinline__ void wave_lds_sync() {
  // LDS accesses of one wave complete in order; this only keeps the compiler from reordering them.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Store rows 0..31 of columns [OFF, OFF + PW) of a staged slab (row-major, pitch kPitch bytes) to C
// at (row_base, col_base + OFF).
template <int PW, int OFF, int kPitch, typename OutT, bool NT>
__device__ __forceinline__ void store_slab_piece(const uint8_t *lds, OutT *__restrict__ C, int64_t ldc, int M, int N,
                                                 int row_base, int col_base, bool vec, int lane) {
  constexpr int ES = (int)sizeof(OutT);
  constexpr int kLanesPerRow = PW * ES / 16;
  constexpr int kRowsPerRead = 64 / kLanesPerRow;
  constexpr int kEl = 16 / ES;  // elements per 16-byte lane access
  static_assert(kLanesPerRow <= 64 && 64 % kLanesPerRow == 0 && 32 % kRowsPerRead == 0, "epilogue piece");
  const int rr = lane / kLanesPerRow, cq = OFF + (lane % kLanesPerRow) * kEl;
  // A piece wholly inside C (the common case) stores without per-lane bounds checks; the test is
  // wave-uniform, so interior tiles never execute the ragged-edge code below.
  const bool interior = vec && (row_base + 31 < M) && (col_base + OFF + PW <= N);
  if (interior) {
    OutT *pc = C + (int64_t)(row_base + rr) * ldc + (col_base + cq);
    // every read of the piece first (one LDS latency), then the stores
    u32x4 vals[32 / kRowsPerRead];
#pragma unroll
    for (int t = 0; t < 32 / kRowsPerRead; ++t)
      vals[t] = *reinterpret_cast<const u32x4 *>(lds + (t * kRowsPerRead + rr) * kPitch + cq * ES);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 32 / kRowsPerRead; ++t) store16<NT>(pc + (int64_t)(t * kRowsPerRead) * ldc, vals[t]);
    return;
  }
#pragma unroll
  for (int t = 0; t < 32 / kRowsPerRead; ++t) {
    const int r = t * kRowsPerRead + rr;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + r * kPitch + cq * ES);
    const int row = row_base + r, col = col_base + cq;
    OutT *pc = C + (int64_t)row * ldc + col;
    if (vec && row < M && col + kEl <= N) {
      store16<NT>(pc, v);
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
}

template <int CW, int TM, int TN, typename OutT, bool NT = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TM][TN], float scale, OutT *__restrict__ C,
                                           int64_t ldc, int M, int N, int row0, int col0, bool vec,
                                           uint8_t *lds, int lane) {
  constexpr int ES = (int)sizeof(OutT);
  constexpr int kPitch = EpiPitch<CW, ES>::kPitch;
  using Pieces = EpiPieces<CW>;
  static_assert(CW == 32 * TN, "epilogue shape");
  const int lr = lane & 31, lh = lane >> 5;
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
    store_slab_piece<Pieces::kFirst, 0, kPitch, OutT, NT>(lds, C, ldc, M, N, row0 + i * 32, col0, vec, lane);
    if constexpr (Pieces::kRest > 0)
      store_slab_piece<Pieces::kRest, Pieces::kFirst, kPitch, OutT, NT>(lds, C, ldc, M, N, row0 + i * 32, col0, vec,
                                                                        lane);
    wave_lds_sync();  // the next slab overwrites this region
  }
}

// ---- NVFP4 output (epilogue-fused requantization) ------------------------------------------------
//
// The GEMM result y = acc * S_A * S_B (+ bias[n]) (-> activation) is computed in fp32 and written
// as NVFP4 under the caller's static tensor scale, with the quantizer's exact rounding rules
// [NVFP4-DiT page, Methodology section 3 (packed operands produced for the next W4A4 product) and
// Definition III.1].  A lane owns one whole 16-column block of one row (the output N is a multiple
// of 16, so a block is wholly inside or wholly outside the matrix).

__device__ __forceinline__ float apply_act(float v, int act) {
  if (act == kActGeluTanh) {
    // GELU, tanh form: 0.5 v (1 + tanh(u)), u = sqrt(2 / pi) (v + 0.044715 v^3).  Evaluated through
    // the identity 0.5 (1 + tanh u) = 1 / (1 + exp(-2 u)) with the hardware exp2 and reciprocal
    // (about 1 ulp each): no cancellation for negative v, and the limits come out exactly
    // (exp -> inf gives v * 0 = -0, exp -> 0 gives v).  exp(-2 u) = 2^(v (c1 + c3 v^2)).
    constexpr float c1 = -1.5957691216057308f * 1.4426950408889634f;
    constexpr float c3 = c1 * 0.044715f;
    const float t = __builtin_amdgcn_exp2f(v * (c1 + c3 * (v * v)));
    return v * __builtin_amdgcn_rcpf(1.0f + t);
  }
  return v;
}

// Requantize and store the 16 values v[0..15] = columns col .. col+15 of `row` (a whole block).
// Branch-light: the common case is decided by the brackets; lanes whose bracket is ambiguous (rare)
// are settled exactly behind one wave-uniform test.
__device__ __forceinline__ void requant16(float (&v)[16], int64_t row, int64_t col, bool valid, int64_t N,
                                          const QuantOut &qo, const QuantConsts &qc) {
  if (qo.bias) {  // uniform; a lane outside the matrix reads column 0 (in bounds) and is not stored
    const f32x4 *bp = reinterpret_cast<const f32x4 *>(qo.bias + (valid ? col : 0));
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 b = bp[h];
      v[4 * h] += b.x;
      v[4 * h + 1] += b.y;
      v[4 * h + 2] += b.z;
      v[4 * h + 3] += b.w;
    }
  }
  if (qo.act == kActGeluTanh) {  // uniform
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = apply_act(v[i], kActGeluTanh);
  }
  if (qo.y) {  // uniform
    if (valid) {
      f32x4 *yp = reinterpret_cast<f32x4 *>(qo.y + row * qo.ldy + col);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 o = {v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
        yp[h] = o;
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  bool amb_b, amb_0, amb_1;
  uint32_t byte = block_byte_fast(amax, qc, amb_b);
  const float inv = __builtin_amdgcn_rcpf(e4m3_to_f32(byte)) * qc.invS;
  const float ilo = byte ? inv * (1.0f - 0x1p-20f) : 0.0f, ihi = byte ? inv * (1.0f + 0x1p-20f) : 0.0f;
  uint32_t c0 = encode8_bracket(v, ilo, ihi, amb_0);
  uint32_t c1 = encode8_bracket(v + 8, ilo, ihi, amb_1);
  const bool exact = valid && (amb_b || amb_0 || amb_1 || !qc.fast_ok);
  if (__builtin_amdgcn_ballot_w64(exact) != 0) {  // rare
    if (exact) {
      byte = block_byte(amax, qc);
      if (byte != 0) {
        c0 = encode_values<8>(v, byte, qc);
        c1 = encode_values<8>(v + 8, byte, qc);
      }
    }
  }
  if (valid) {
    const u32x2 o = {c0, c1};
    *reinterpret_cast<u32x2 *>(qo.packed + row * (N / 2) + col / 2) = o;
    qo.scales[row * (N / 16) + col / 16] = (uint8_t)byte;
  }
}

// Requantize rows 0..31 of columns [OFF, OFF + PW) of a staged fp32 slab: each lane reads back one
// whole 16-column block of a row.
template <int PW, int OFF, int kPitch>
__device__ __forceinline__ void requant_slab_piece(const uint8_t *lds, const QuantOut &qo, const QuantConsts &qc,
                                                   int M, int N, int row_base, int col_base, int lane) {
  constexpr int kLanesPerRow = PW / 16;
  constexpr int kRowsPerRead = 64 / kLanesPerRow;
  static_assert(64 % kLanesPerRow == 0 && 32 % kRowsPerRead == 0, "epilogue piece");
  const int rr = lane / kLanesPerRow, cb = OFF + (lane % kLanesPerRow) * 16;
  // not unrolled: a short slab body lets the slab loop unroll, so the accumulators are only ever
  // indexed at compile time (no copy in scratch memory)
#pragma unroll 1
  for (int t = 0; t < 32 / kRowsPerRead; ++t) {
    const int r = t * kRowsPerRead + rr;
    float v[16];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 q = *reinterpret_cast<const f32x4 *>(lds + r * kPitch + (cb + 4 * h) * 4);
      v[4 * h] = q.x;
      v[4 * h + 1] = q.y;
      v[4 * h + 2] = q.z;
      v[4 * h + 3] = q.w;
    }
    const int row = row_base + r, col = col_base + cb;
    requant16(v, row, col, row < M && col < N, N, qo, qc);
  }
}

// store_tile for NVFP4 output: the wave's sub-tile goes through the same padded row-major fp32
// staging as store_tile, then is requantized block by block.
template <int CW, int TM, int TN>
__device__ __forceinline__ void store_tile_nvfp4(const f32x16 (&acc)[TM][TN], float scale, const QuantOut &qo,
                                                 int M, int N, int row0, int col0, uint8_t *lds, int lane) {
  constexpr int kPitch = EpiPitch<CW, 4>::kPitch;
  using Pieces = EpiPieces<CW>;
  static_assert(CW == 32 * TN, "epilogue shape");
  const QuantConsts qc = make_quant_consts(*qo.out_ts, false);
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 o = {__float_as_uint(acc[i][j][4 * g] * scale), __float_as_uint(acc[i][j][4 * g + 1] * scale),
                         __float_as_uint(acc[i][j][4 * g + 2] * scale), __float_as_uint(acc[i][j][4 * g + 3] * scale)};
        *reinterpret_cast<u32x4 *>(lds + lr * kPitch + (j * 32 + 8 * g + 4 * lh) * 4) = o;
      }
    }
    wave_lds_sync();
    requant_slab_piece<Pieces::kFirst, 0, kPitch>(lds, qo, qc, M, N, row0 + i * 32, col0, lane);
    if constexpr (Pieces::kRest > 0)
      requant_slab_piece<Pieces::kRest, Pieces::kFirst, kPitch>(lds, qo, qc, M, N, row0 + i * 32, col0, lane);
    wave_lds_sync();  // the next slab overwrites this region
  }
}

}  // namespace nvfp4
