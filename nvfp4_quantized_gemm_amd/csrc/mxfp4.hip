// MXFP4 for gfx950: 32-value blocks with a power-of-two E8M0 scale (the OCP microscaling format;
// the vllm-omni NVFP4 RFC names MXFP4 as the related format, Motivation).  Quantize, dequantize and
// a GEMM on CDNA4's block-scaled FP4 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Definition: per block, X = 2^(floor(log2 amax) - 2) clamped to 2^-127 (byte 0 also for an
// all-zero block); each value becomes the E2M1 value nearest to v / X, ties to the even code,
// clipped to +-6, sign copied.  With b the E8M0 byte, floor(log2 amax) + 127 is amax's exponent
// field E, so b = max(E - 2, 0); v * 2^(127 - b) is exact (a power-of-two scaling whose result is
// below 8), and the hardware E2M1 conversion (round-half-even, saturating, sign-preserving) of that
// exact value is the code: no bracketing is needed.  Dequantize: y = q * 2^(b - 127), exact in fp32
// for every byte the quantizer produces.
//
// GEMM: the matrix instruction takes, per lane l (row l % 32, k-half l / 32 of a 64-k step), 16
// bytes holding 32 E2M1 codes low nibble first -- exactly 16 contiguous bytes of a canonical packed
// row -- and one E8M0 byte per lane (its row's 32-value block) selected by op_sel.  Both operands
// are therefore streamed straight from the canonical layout into LDS by LDS-DMA; no prepack and no
// dequantization.  The products q_a X_a q_b X_b are exact in fp32 and accumulate in fp32.
#include <type_traits>

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kMxBlk = 32;
constexpr int kMxSegsPerLane = 4;

__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {  // amax >= 0, finite
  const uint32_t E = (__float_as_uint(amax) >> 23) & 0xffu;
  return E >= 2u ? E - 2u : 0u;
}
// 2^(127 - b) for b <= 252: maps the block onto the E2M1 grid exactly
__device__ __forceinline__ float mx_inv_scale(uint32_t b) { return __uint_as_float((254u - b) << 23); }
// X = 2^(b - 127) as fp32 (2^-127 is the subnormal 0x00400000)
__device__ __forceinline__ float mx_scale_value(uint32_t b) { return __uint_as_float(b ? (b << 23) : 0x00400000u); }

int mx_grid(uint64_t nseg, int cap) {
  const uint64_t tiles = (nseg + 64 * kMxSegsPerLane - 1) / (64 * kMxSegsPerLane);
  uint64_t g = (tiles + 3) / 4;
  if (g < 1) g = 1;
  return (int)(g > (uint64_t)cap ? (uint64_t)cap : g);
}

}  // namespace

// ---- quantize: lane-contiguous 16-byte segments, 4 (bf16) or 8 (fp32) lanes per 32-value block ----

template <int DT, bool DENSE>
__global__ __launch_bounds__(256) void k_mx_quantize(const void *__restrict__ x, int64_t ld, uint64_t nseg,
                                                     FastDiv bpr, uint8_t *__restrict__ packed,
                                                     uint8_t *__restrict__ scales) {
  using In = SegIn<DT>;
  constexpr int E = In::kElems;
  using Map = Segments<E, kMxBlk>;
  constexpr int U = kMxSegsPerLane;
  const int lane = threadIdx.x & 63;
  const uint64_t ntiles = (nseg + 64 * U - 1) / (64 * U);
  const uint64_t tstride = gridDim.x * 4ull;
  auto fetch = [&](uint64_t t, u32x4 *r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t g = t * (64 * U) + u * 64 + lane;
      g = g < nseg ? g : nseg - 1;
      r[u] = In::template raw<true>(x, Map::template offset<DENSE>(g, bpr, ld));  // streaming: read once
    }
  };
  uint64_t t = blockIdx.x * 4ull + (threadIdx.x >> 6);
  u32x4 nxt[U];
  if (t < ntiles) fetch(t, nxt);
  for (; t < ntiles; t += tstride) {
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    if (t + tstride < ntiles) fetch(t + tstride, nxt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t g = t * (64 * U) + u * 64 + lane;
      float v[E];
      In::unpack(cur[u], v);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(v[i]));
      amax = fmaxf(amax, swap_lane1(amax));
      amax = fmaxf(amax, swap_lane2(amax));
      if (Map::kLanesPerBlock == 8) amax = fmaxf(amax, swap_lane4(amax));
      if (g >= nseg) continue;  // whole blocks are in or out of range
      const uint32_t b = mx_scale_byte(amax);
      const float m = mx_inv_scale(b);
      uint32_t codes = 0;
      codes = fp4_encode2<0>(codes, v[0] * m, v[1] * m);
      codes = fp4_encode2<1>(codes, v[2] * m, v[3] * m);
      if (E == 8) {
        codes = fp4_encode2<2>(codes, v[4] * m, v[5] * m);
        codes = fp4_encode2<3>(codes, v[6] * m, v[7] * m);
        *reinterpret_cast<uint32_t *>(packed + 4 * g) = codes;
      } else {
        *reinterpret_cast<uint16_t *>(packed + 2 * g) = (uint16_t)codes;
      }
      if ((lane & (Map::kLanesPerBlock - 1)) == 0) scales[g >> Map::kShift] = (uint8_t)b;
    }
  }
}

// ---- dequantize: y = q * X ----------------------------------------------------------------------------

template <int OUT, bool DENSE>
__global__ __launch_bounds__(256) void k_mx_dequantize(const uint8_t *__restrict__ packed,
                                                       const uint8_t *__restrict__ scales, uint64_t nseg,
                                                       FastDiv bpr, void *__restrict__ y, int64_t ld_y) {
  constexpr int E = (OUT == 1) ? 8 : 4;
  using Map = Segments<E, kMxBlk>;
  constexpr int U = kMxSegsPerLane;
  const int lane = threadIdx.x & 63;
  const uint64_t ntiles = (nseg + 64 * U - 1) / (64 * U);
  for (uint64_t t = blockIdx.x * 4ull + (threadIdx.x >> 6); t < ntiles; t += gridDim.x * 4ull) {
    uint32_t codes[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t g = t * (64 * U) + u * 64 + lane;
      g = g < nseg ? g : nseg - 1;
      codes[u] = (E == 8) ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(packed + 4 * g))
                          : (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(packed + 2 * g));
      sb[u] = scales[g >> Map::kShift];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t g = t * (64 * U) + u * 64 + lane;
      if (g >= nseg) break;
      const float X = mx_scale_value(sb[u]);
      float out[E];
      const f32x2 q0 = fp4_decode2_f32<0>(codes[u]), q1 = fp4_decode2_f32<1>(codes[u]);
      out[0] = q0.x * X;
      out[1] = q0.y * X;
      out[2] = q1.x * X;
      out[3] = q1.y * X;
      if (E == 8) {
        const f32x2 q2 = fp4_decode2_f32<2>(codes[u]), q3 = fp4_decode2_f32<3>(codes[u]);
        out[4] = q2.x * X;
        out[5] = q2.y * X;
        out[6] = q3.x * X;
        out[7] = q3.y * X;
      }
      const uint64_t off = Map::template offset<DENSE>(g, bpr, ld_y);
      u32x4 o;
      if (OUT == 0) {
        o.x = __float_as_uint(out[0]);
        o.y = __float_as_uint(out[1]);
        o.z = __float_as_uint(out[2]);
        o.w = __float_as_uint(out[3]);
        store16<true>(static_cast<float *>(y) + off, o);  // streaming: written once
      } else {
        uint32_t p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 h = {(__bf16)out[2 * j], (__bf16)out[2 * j + 1]};
          p[j] = __builtin_bit_cast(uint32_t, h);
        }
        o.x = p[0];
        o.y = p[1];
        o.z = p[2];
        o.w = p[3];
        store16<true>(static_cast<uint16_t *>(y) + off, o);
      }
    }
  }
}

// ---- GEMM: Y[M][N] = A[M][K] B[N][K]^T, both operands canonical MXFP4 ---------------------------------
//
// T x T tile per workgroup of WM x WN waves, each owning (T / WM) x (T / WN) = TM x TN tiles of
// 32 x 32.  T = 256: 2 x 4 waves (two per SIMD, 128 x 64 each, so one wave's LDS and DMA waits
// overlap the other's MFMAs), one workgroup per CU.  T = 128: 2 x 2 waves of 64 x 64, two
// workgroups per CU.  K in chunks of 128 (two 64-k MFMA steps).  LDS stage (T / 8 KB):
//   A codes  [T / 16 blocks of 16 rows][4 pieces][16 rows][16 B]   B codes likewise (columns).
// A codes block holds 16 rows x the chunk's 64 bytes each, piece-major, so one DMA reads whole
// 64-byte row segments and every 16-lane LDS read pass is contiguous; MFMA lane (r, h) of step s
// reads piece 2 s + h of row r (k-half h of the step).  A 4-stage ring with the DMA three chunks
// ahead and the next chunk's fragments read into registers during the current chunk's MFMAs; one
// barrier per chunk.
// Scales come in blocks of 4 chunks, double-buffered beside the ring: a row's scale word of a
// chunk (its 4 bytes, 4-byte aligned in the canonical [rows][K/32] layout) is one 4-byte
// DMA lane, and one DMA covers 16 rows x 4 chunks (lane = 16 * chunk + row), so an operand's T
// rows take T / 16 DMAs per 4 chunks:  scale block [T / 16 row blocks][4 chunks][16 rows][4 B].  Block
// j + 1 is issued in the first chunk of block j, after that chunk's codes, and is needed from the
// look-ahead read of chunk 4 j + 4 on (three chunks later); the chunk waits account for it.  When
// K % 512 == 0 and both scale arrays are 16-byte aligned, rows of scales are 16-byte aligned and a
// row's 4 words of a block are one 16-byte DMA lane instead (SX = 4: T / 64 DMAs per operand per
// block, block layout [T rows][4 chunks][4 B]).  Of a
// word, block 2 s + h feeds the MFMA: the lane shifts the word right by 8 h and op_sel picks byte
// 2 s.  Rows past M / N are clamped to the last one (never stored), chunks past K to the last.
#ifndef MX_WM
#define MX_WM 2
#endif
#ifndef MX_WN
#define MX_WN 4
#endif

namespace {
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i as_v8(const u32x4 &v) {
  const v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

// One 32x32x64 block-scaled FP4 MFMA of step T: op_sel 2T picks scale byte 2T of each lane's word.
template <int T>
__device__ __forceinline__ f32x16 mx_mfma(const u32x4 &row_op, const u32x4 &col_op, const f32x16 &c, uint32_t s_row,
                                          uint32_t s_col) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8(row_op), as_v8(col_op), c, 4, 4, 2 * T, (int)s_row,
                                                         2 * T, (int)s_col);
}

// LDS byte offset of lane (r, h)'s 16-byte operand of step t in row group grp: row r's piece
// 2 t + h sits in codes block 2 grp + r / 16 at slot 16 (2 t + h) + r % 16, so a 16-lane read pass
// is one contiguous 256-byte span (conflict-free).
__device__ __forceinline__ int frag_off(int grp, int t, int lane) {
  const int r = lane & 31, h = lane >> 5;
  return (2 * grp + (r >> 4)) * 1024 + (16 * (2 * t + h) + (r & 15)) * 16;
}

// T x T tile (T = 256 or 128) of WM x WN waves
template <int T, int WM, int WN, int SX>
struct MxCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kTM = T / 32 / WM, kTN = T / 32 / WN;  // 32 x 32 tiles per wave
  static constexpr int kBlocks = T / 16;                      // 16-row blocks per operand
  static constexpr int kCodes = kBlocks * 1024;               // one operand's codes of a chunk
  static constexpr int kStage = 2 * kCodes;
  static constexpr int kStages = 4;
  static constexpr int kScaleBlk = 16 * T;                    // one operand's scale words of 4 chunks
  static constexpr int kScaleBase = kStages * kStage;         // [2 slots][A, B][kScaleBlk]
  static constexpr int kLds = kScaleBase + 2 * 2 * kScaleBlk;
  // DMA loads per wave: codes T / 16 per operand per chunk; scales per 4 chunks T / 16 per operand
  // with one word per lane (SX = 1), or T / 64 per operand with a row's 4 words per lane (SX = 4)
  static constexpr int kQ4 = T / 64;
  static constexpr int kNC = kBlocks / kWaves, kNS = kBlocks / kWaves, kNS4 = 2 * kQ4 / kWaves;
  static constexpr int kSlots = 2 * kNC;                       // per chunk
  static constexpr int kSSlots = (SX == 1) ? 2 * kNS : kNS4;   // per scale block
  static_assert(kNC * kWaves == kBlocks && kNS4 * kWaves == 2 * kQ4, "even DMA split");
  static_assert(kTM * WM * 32 == T && kTN * WN * 32 == T, "wave tiling");
  static_assert(SX == 1 || SX == 4, "scale words per DMA lane");
  static_assert(kLds <= 160 * 1024, "LDS fits");
};
}  // namespace

// waves per SIMD: one 256-tile workgroup per CU (2 x 4 waves: two per SIMD), or two 128-tile
// workgroups of 2 x 2 waves
template <int T, int WM, int WN>
constexpr int mx_waves_per_eu() { return T == 256 ? WM * WN / 4 : 2 * WM * WN / 4; }

template <int OUT, int T, int WM, int WN, int SX>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(mx_waves_per_eu<T, WM, WN>(), mx_waves_per_eu<T, WM, WN>()))) void k_mx_gemm(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ as, const uint8_t *__restrict__ b,
    const uint8_t *__restrict__ bs, int M, int N, int K, void *__restrict__ c, int64_t ldc, int tiles_m,
    int tiles_n) {
  using Cfg = MxCfg<T, WM, WN, SX>;
  constexpr int TM = Cfg::kTM, TN = Cfg::kTN, S = Cfg::kStages, W = Cfg::kWaves;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lh = lane >> 5;

  // XCD-aware grouped tile order (bijective on the multiple-of-8 prefix), as in the NVFP4 GEMM
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int full = (ntiles / 8) * 8;
    if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  }
  int tmi, tni;
  grouped_tile<4>(bid, tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * T, n0 = tni * T;
  const int nk = K / 128;
  const uint32_t rowb = (uint32_t)(K / 2), srow = (uint32_t)(K / 32);  // bytes per codes / scales row

  // DMA sources: wave-uniform tile bases + 32-bit lane offsets (host: T * rowb < 2^31)
  const uint8_t *a_tile = a + (int64_t)m0 * rowb, *as_tile = as + (int64_t)m0 * srow;
  const uint8_t *b_tile = b + (int64_t)n0 * rowb, *bs_tile = bs + (int64_t)n0 * srow;
  uint32_t oa[Cfg::kNC], ob[Cfg::kNC];
  uint32_t oas[SX == 1 ? Cfg::kNS : 1], obs[SX == 1 ? Cfg::kNS : 1], osx[SX == 4 ? Cfg::kNS4 : 1];
#pragma unroll
  for (int i = 0; i < Cfg::kNC; ++i) {
    // codes block d covers rows 16 d .. 16 d + 15 with all 64 bytes of each: lane l takes row
    // 16 d + l % 16, 16-byte piece l / 16 (so a DMA touches 16 rows x 64 B, not 32 rows x 32 B)
    const int d = wave + W * i, row16 = 16 * d + (lane & 15), piece = lane >> 4;
    oa[i] = (uint32_t)(min(m0 + row16, M - 1) - m0) * rowb + 16 * piece;
    ob[i] = (uint32_t)(min(n0 + row16, N - 1) - n0) * rowb + 16 * piece;
  }
  if constexpr (SX == 1) {
#pragma unroll
    for (int i = 0; i < Cfg::kNS; ++i) {
      // scale DMA d covers rows 16 d .. 16 d + 15: lane l takes row 16 d + l % 16, chunk l / 16 of the block
      const int row16 = 16 * (wave + W * i) + (lane & 15);
      oas[i] = (uint32_t)(min(m0 + row16, M - 1) - m0) * srow;
      obs[i] = (uint32_t)(min(n0 + row16, N - 1) - n0) * srow;
    }
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::kNS4; ++i) {
      // scale DMA q (0 .. 2 T / 64 - 1) covers operand q / (T / 64), rows 64 (q % (T / 64)) .. + 63,
      // one row per lane
      const int q = wave + W * i, row64 = 64 * (q % Cfg::kQ4) + lane;
      osx[i] = (q / Cfg::kQ4) ? (uint32_t)(min(n0 + row64, N - 1) - n0) * srow
                              : (uint32_t)(min(m0 + row64, M - 1) - m0) * srow;
    }
  }
  auto issue = [&](int kc, int stage) {
    uint8_t *st = smem + stage * Cfg::kStage;
#pragma unroll
    for (int i = 0; i < Cfg::kNC; ++i) g2l16(a_tile + (int64_t)kc * 64 + oa[i], st + (wave + W * i) * 1024);
#pragma unroll
    for (int i = 0; i < Cfg::kNC; ++i)
      g2l16(b_tile + (int64_t)kc * 64 + ob[i], st + Cfg::kCodes + (wave + W * i) * 1024);
  };
  // scale block blk (chunks 4 blk .. 4 blk + 3, clamped to the last chunk) into slot blk % 2;
  // 32-bit lane offsets on the wave-uniform tile bases
  auto issue_scales = [&](int blk) {
    uint8_t *sl = smem + Cfg::kScaleBase + (blk & 1) * (2 * Cfg::kScaleBlk);
    if constexpr (SX == 1) {
      const uint32_t kcw = (uint32_t)min(4 * blk + (lane >> 4), nk - 1) * 4u;
#pragma unroll
      for (int i = 0; i < Cfg::kNS; ++i) g2l4(as_tile + (oas[i] + kcw), sl + (wave + W * i) * 256);
#pragma unroll
      for (int i = 0; i < Cfg::kNS; ++i) g2l4(bs_tile + (obs[i] + kcw), sl + Cfg::kScaleBlk + (wave + W * i) * 256);
    } else {
      // nk % 4 == 0 here: blocks are whole; the look-ahead past the last block re-reads the last
      const uint32_t kcw = (uint32_t)min(blk, nk / 4 - 1) * 16u;
#pragma unroll
      for (int i = 0; i < Cfg::kNS4; ++i) {
        const int q = wave + W * i, op = q / Cfg::kQ4;
        g2l16((op ? bs_tile : as_tile) + (osx[i] + kcw), sl + op * Cfg::kScaleBlk + (q % Cfg::kQ4) * 1024);
      }
    }
  };

  u32x4 Af[2][TM][2], Bf[2][TN][2];
  uint32_t Sa[2][TM], Sb[2][TN];
  // fragments and scale words of chunk kc (held in ring stage `stage`) into register buffer buf;
  // row lr of row group grp has its word in scale row block 2 grp + lr / 16 at lane 16 (kc % 4) + lr % 16
  auto read_frags = [&](int stage, int buf, int kc) {
    const uint8_t *st = smem + stage * Cfg::kStage;
    // SX = 1: row lr's word at row block 2 grp + lr / 16, lane 16 (kc % 4) + lr % 16;
    // SX = 4: at row 32 grp + lr, word kc % 4 (16 bytes per row)
    const uint8_t *sc = smem + Cfg::kScaleBase + ((kc >> 2) & 1) * (2 * Cfg::kScaleBlk) +
                        ((SX == 1) ? ((lane >> 4) & 1) * 256 + ((kc & 3) * 16 + (lane & 15)) * 4
                                   : (lane & 31) * 16 + (kc & 3) * 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int grp = wm * TM + i;
#pragma unroll
      for (int t = 0; t < 2; ++t) Af[buf][i][t] = *reinterpret_cast<const u32x4 *>(st + frag_off(grp, t, lane));
      Sa[buf][i] = *reinterpret_cast<const uint32_t *>(sc + grp * 512);
    }
    const uint8_t *sb = st + Cfg::kCodes;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int grp = wn * TN + j;
#pragma unroll
      for (int t = 0; t < 2; ++t) Bf[buf][j][t] = *reinterpret_cast<const u32x4 *>(sb + frag_off(grp, t, lane));
      Sb[buf][j] = *reinterpret_cast<const uint32_t *>(sc + Cfg::kScaleBlk + grp * 512);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Branch-free pipeline: near the end of K the DMA re-fetches the last chunk into the free stage
  // and the look-ahead reads a stale stage; neither result is used.
  issue_scales(0);
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(min(s, nk - 1), s);
  wait_vmem_then_barrier<(S - 2) * Cfg::kSlots>();  // scale block 0 and chunk 0 landed
  read_frags(0, 0, 0);
  // one chunk; CUR (compile time) is the register buffer holding its fragments, P = kc % 4.  In
  // issue order the DMAs are: chunk kc + 3's codes per chunk, and after them in phase 0 the scale
  // block kc / 4 + 1.  "Chunk kc + 1 landed" therefore leaves one chunk's codes outstanding in
  // phases 0 and 3 and also the scale block in phases 1 and 2; in phase 3 the scale block issued
  // in phase 0 is thereby complete before the look-ahead reads chunk kc + 1 (its first chunk).
  auto chunk = [&](int kc, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    const int P = kc & 3;  // wave-uniform: the branches below are scalar
    if (P == 1 || P == 2) wait_vmem_then_barrier<(S - 3) * Cfg::kSlots + Cfg::kSSlots>();
    else wait_vmem_then_barrier<(S - 3) * Cfg::kSlots>();
    // this chunk's scale words (read one chunk ago): lane (r, h) feeds blocks h and 2 + h, i.e.
    // bytes 0 and 2 after a shift by 8 h.  Done before the next reads are issued, so waiting for
    // the old reads does not wait for the new ones.
#pragma unroll
    for (int i = 0; i < TM; ++i) Sa[CUR][i] >>= 8 * lh;
#pragma unroll
    for (int j = 0; j < TN; ++j) Sb[CUR][j] >>= 8 * lh;
    __builtin_amdgcn_sched_barrier(0);
    issue(min(kc + S - 1, nk - 1), (kc + S - 1) % S);   // into the stage chunk kc-1 used
    if (P == 0) issue_scales(kc / 4 + 1);                 // into the slot block kc / 4 - 1 used
    read_frags((kc + 1) % S, CUR ^ 1, kc + 1);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mx_mfma<0>(Bf[CUR][j][0], Af[CUR][i][0], acc[i][j], Sb[CUR][j], Sa[CUR][i]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mx_mfma<1>(Bf[CUR][j][1], Af[CUR][i][1], acc[i][j], Sb[CUR][j], Sa[CUR][i]);
  };
  int kc = 0;
  for (; kc + 1 < nk; kc += 2) {
    chunk(kc, std::integral_constant<int, 0>{});
    chunk(kc + 1, std::integral_constant<int, 1>{});
  }
  if (kc < nk) chunk(kc, std::integral_constant<int, 0>{});

  wait_vmem();      // the last look-ahead DMA targets the ring, which now stages output
  __syncthreads();
  typedef typename std::conditional<OUT == 0, float, __bf16>::type OutT;
  const bool vec = (ldc * (int64_t)sizeof(OutT)) % 16 == 0;
  constexpr int CW = T / WN;  // columns per wave
  static_assert(W * 32 * EpiPitch<CW, 4>::kPitch <= S * Cfg::kStage, "epilogue staging fits the LDS ring");
  uint8_t *lds_wave = smem + wave * (32 * EpiPitch<CW, 4>::kPitch);
  store_tile<CW, TM, TN, OutT, true>(acc, 1.0f, static_cast<OutT *>(c), ldc, M, N, m0 + wm * (T / WM), n0 + wn * CW,
                                     vec, lds_wave, lane);
}

// Generic fallback (any K % 32 == 0): one thread per output element.
template <int OUT>
__global__ __launch_bounds__(256) void k_mx_gemm_generic(const uint8_t *__restrict__ a, const uint8_t *__restrict__ as,
                                                         const uint8_t *__restrict__ b, const uint8_t *__restrict__ bs,
                                                         int64_t M, int64_t N, int64_t K, void *__restrict__ c,
                                                         int64_t ldc) {
  for (int64_t t = blockIdx.x * 256ll + threadIdx.x; t < M * N; t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / N, n = t % N;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const uint32_t ca = (a[m * (K / 2) + k / 2] >> (4 * (k & 1))) & 15u;
      const uint32_t cb = (b[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15u;
      const float xa = fp4_decode2_f32<0>(ca).x * mx_scale_value(as[m * (K / 32) + k / 32]);
      const float xb = fp4_decode2_f32<0>(cb).x * mx_scale_value(bs[n * (K / 32) + k / 32]);
      acc = fmaf(xa, xb, acc);
    }
    if (OUT == 0) static_cast<float *>(c)[m * ldc + n] = acc;
    else static_cast<__bf16 *>(c)[m * ldc + n] = (__bf16)acc;
  }
}

// ---- launchers --------------------------------------------------------------------------------------

hipError_t launch_mx_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, uint8_t *packed,
                              uint8_t *scales, hipStream_t stream) {
  const FastDiv bpr = make_fastdiv((uint32_t)(K / kMxBlk));
  const uint64_t nseg = (uint64_t)M * (uint64_t)K / (dtype == 0 ? 4u : 8u);
  const int grid = mx_grid(nseg, kMxQuantizeMaxGrid);
  const bool dense = (ld == K);
  if (dtype == 0) {
    if (dense) k_mx_quantize<0, true><<<grid, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales);
    else k_mx_quantize<0, false><<<grid, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales);
  } else {
    if (dense) k_mx_quantize<1, true><<<grid, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales);
    else k_mx_quantize<1, false><<<grid, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales);
  }
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, void *y,
                                int out_dtype, int64_t ld_y, hipStream_t stream) {
  const FastDiv bpr = make_fastdiv((uint32_t)(K / kMxBlk));
  const uint64_t nseg = (uint64_t)M * (uint64_t)K / (out_dtype == 0 ? 4u : 8u);
  const int grid = mx_grid(nseg, kDequantizeMaxGrid);
  const bool dense = (ld_y == K);
  if (out_dtype == 0) {
    if (dense) k_mx_dequantize<0, true><<<grid, 256, 0, stream>>>(packed, scales, nseg, bpr, y, ld_y);
    else k_mx_dequantize<0, false><<<grid, 256, 0, stream>>>(packed, scales, nseg, bpr, y, ld_y);
  } else {
    if (dense) k_mx_dequantize<1, true><<<grid, 256, 0, stream>>>(packed, scales, nseg, bpr, y, ld_y);
    else k_mx_dequantize<1, false><<<grid, 256, 0, stream>>>(packed, scales, nseg, bpr, y, ld_y);
  }
  return hipGetLastError();
}

template <int OUT, int T, int WM, int WN, int SX>
static hipError_t launch_mx_tiled(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int64_t M,
                                  int64_t N, int64_t K, void *c, int64_t ldc, hipStream_t stream) {
  using Cfg = MxCfg<T, WM, WN, SX>;
  const int tm = (int)((M + T - 1) / T), tn = (int)((N + T - 1) / T);
  constexpr int smem = Cfg::kLds;
  static std::atomic<bool> configured[kMaxDevices];  // per instantiation and device
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(k_mx_gemm<OUT, T, WM, WN, SX>), smem, configured);
  if (e != hipSuccess) return e;
  k_mx_gemm<OUT, T, WM, WN, SX><<<tm * tn, Cfg::kWaves * 64, smem, stream>>>(a, as, b, bs, (int)M, (int)N, (int)K, c,
                                                                            ldc, tm, tn);
  return hipGetLastError();
}

// Tile choice: 128 x 128 tiles (up to two workgroups per CU) when 256 x 256 tiles (one per CU)
// would leave CUs idle and the small tiles still fit one round, i.e. at most two per CU of the
// chip's 256.  A lone 128-tile workgroup runs a chunk in ~0.56x the time of a 256-tile one for a
// quarter of the work, so the small tiles win only by occupying more CUs (4096 x 1152 x 1152:
// 14.3 -> 11.0 us, 2048^3: 21.7 -> 12.1 us) and lose once they need more than one round (4096 x
// 3456 x 1152, 864 tiles: 18.7 -> 21.7 us).
static bool mx_use_small_tiles(int64_t M, int64_t N) {
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  return t256 < 256 && t128 <= 2 * 256;
}

template <int OUT>
static hipError_t launch_mx_gemm_out(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs,
                                     int64_t M, int64_t N, int64_t K, void *c, int64_t ldc, hipStream_t stream) {
  if (K % 128 != 0 || 256 * (K / 2) >= (int64_t(1) << 31)) {
    int64_t grid = (M * N + 255) / 256;
    if (grid > 65536) grid = 65536;
    k_mx_gemm_generic<OUT><<<(unsigned)grid, 256, 0, stream>>>(a, as, b, bs, M, N, K, c, ldc);
    return hipGetLastError();
  }
  // a row's 4 scale words of a 4-chunk block are one 16-byte DMA lane when rows (K / 32 bytes)
  // and both scale arrays are 16-byte aligned
  const bool sx4 = K % 512 == 0 && reinterpret_cast<uintptr_t>(as) % 16 == 0 && reinterpret_cast<uintptr_t>(bs) % 16 == 0;
  auto small = [&](const uint8_t *bb, const uint8_t *bbs, int64_t n, void *cc) {
    return sx4 ? launch_mx_tiled<OUT, 128, 2, 2, 4>(a, as, bb, bbs, M, n, K, cc, ldc, stream)
               : launch_mx_tiled<OUT, 128, 2, 2, 1>(a, as, bb, bbs, M, n, K, cc, ldc, stream);
  };
  auto big = [&](int64_t n) {
    return sx4 ? launch_mx_tiled<OUT, 256, MX_WM, MX_WN, 4>(a, as, b, bs, M, n, K, c, ldc, stream)
               : launch_mx_tiled<OUT, 256, MX_WM, MX_WN, 1>(a, as, b, bs, M, n, K, c, ldc, stream);
  };
  if (mx_use_small_tiles(M, N)) return small(b, bs, N, c);
  // More than one round of 256 x 256 tiles: when the columns that make exactly one round leave a
  // remainder of at most one 128 x 128 tile per CU, run that remainder as a second launch of
  // small tiles instead of a second, mostly idle round of big ones.  B and C of the remainder are
  // the same arrays from column n_big on (B rows and scale rows are whole rows).
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, cols = 256 / tm;
  if (tm * tn > 256 && cols >= 1 && cols < tn) {
    const int64_t n_big = cols * 256;
    const int64_t rest = ((M + 127) / 128) * ((N - n_big + 127) / 128);
    if (rest <= 256) {
      hipError_t e = big(n_big);
      if (e != hipSuccess) return e;
      const size_t esz = OUT == 0 ? 4 : 2;
      return small(b + n_big * (K / 2), bs + n_big * (K / 32), N - n_big, static_cast<uint8_t *>(c) + n_big * esz);
    }
  }
  return big(N);
}

hipError_t launch_mx_gemm(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int64_t M,
                          int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc, hipStream_t stream) {
  return out_dtype == 0 ? launch_mx_gemm_out<0>(a, as, b, bs, M, N, K, c, ldc, stream)
                        : launch_mx_gemm_out<1>(a, as, b, bs, M, N, K, c, ldc, stream);
}

}  // namespace nvfp4
