// NVFP4 GEMM for gfx950: Y[M][N] = A[M][K] * B[N][K]^T with B an NVFP4 weight in the prepacked
// layout (prepack.hip) and A either NVFP4 (W4A4, canonical layout from the quantizer) or bf16
// (W4A16) [NVFP4-DiT page, Methodology section 3: packed operands dequantized on the fly, FP32
// accumulation; vllm-omni NVFP4 RFC, Open Question 1: W4A4 and weight-only W4A16].
//
// Why 16-bit matrix-core operands: each dequantized factor q * e has at most 2 + 4 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16 and in bf16, and every product of two such
// factors is exact in the fp32 accumulator; only the summation order differs from the
// dequantize-then-matmul definition.  gfx950's block-scaled FP4/FP8 MFMA takes one power-of-two
// (E8M0) scale per 32 k, which cannot represent an E4M3 scale per 16 k, and q * e is not exact in
// FP8; so the exact route is fp16 (W4A4) / bf16 (W4A16, where A is bf16) MFMA.
//
// Kernel structure (k_gemm_tiled): a 256-thread workgroup (4 waves) owns a BM x BN tile (W4A4:
// 256 x 256, 128 x 128 or 128 x 192; W4A16: 128 x 256 or 64 x 256) and walks K in chunks of 128.
// Per chunk, LDS-DMA loads stage A codes + A scale bytes (or bf16 A) and one prepacked B unit per
// 32 columns into a three-stage LDS ring, two chunks ahead of the MFMAs (one barrier per chunk).
// Each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  For MFMA step s
// (16 k) lane l = r + 32 h takes k in [64 h + 8 s, +8): that is dword s of the lane's 32-byte code
// run, so A and B codes are read with 16-byte LDS loads and the k permutation is the same on both
// sides.  Dequantization in registers: v_cvt_scalef32_pk_{f16,f32}_fp4 with scale 1 gives exact q;
// one multiply by the block's E4M3 scale gives q * e.  The epilogue multiplies the fp32
// accumulator by S_A * S_B and converts.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kChunk = 128;  // k per LDS stage
constexpr bool kOutputNT = true;    // streaming stores for the bf16 / fp32 output
constexpr bool kPartialNT = false;  // split-K partials (read back at once by the reduction)
constexpr bool kReduceNT = false;   // the reduction reads the partials while they are still cached

// HS: W4A16 stages half chunks (64 k, one part of the prepacked units), so that a 128 x 256
// workgroup's three stages take 78 KB of LDS and two workgroups fit on a CU.
template <int MODE, int BM, int BN, bool HS>
struct TileCfg {
  static_assert(!HS || MODE == 1, "half-chunk stages are a W4A16 form");
  static constexpr bool kHalf = HS;
  static constexpr int kALds = (MODE == 0) ? BM * 64 : (kHalf ? BM * 128 : BM * 256);  // codes or bf16
  static constexpr int kASLds = (MODE == 0) ? BM * 8 : 0;
  static constexpr int kBLds = kHalf ? BN * 32 : BN * 64;
  // B scale blocks (256 B per 32-column unit) come one per wave per DMA round, so their count is
  // rounded up to a multiple of the 4 waves: a 192-column tile also fetches the next two units
  // (clamped to the matrix), whose bytes are never read
  static constexpr int kBSUnits = (BN / 32 + 3) / 4 * 4;
  static constexpr int kBSLds = kBSUnits * 256;
  static constexpr int kStage = kALds + kASLds + kBLds + kBSLds;
};

// exact E2M1 decode of the 8 codes of a dword (element 2j in the low nibble of byte j)
__device__ __forceinline__ f16x8 decode_f16x8(uint32_t codes) {
  const f16x2 q[4] = {fp4_decode2_f16<0>(codes), fp4_decode2_f16<1>(codes), fp4_decode2_f16<2>(codes),
                      fp4_decode2_f16<3>(codes)};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = q[j].x;
    r[2 * j + 1] = q[j].y;
  }
  return r;
}

__device__ __forceinline__ f16x8 scale_f16x8(const f16x8 &q, _Float16 e) {
  const f16x8 ee = {e, e, e, e, e, e, e, e};
  return q * ee;  // q * e is exact in fp16
}

__device__ __forceinline__ bf16x8 dequant_bf16x8(uint32_t codes, float e) {
  const f32x2 q[4] = {fp4_decode2_f32<0>(codes), fp4_decode2_f32<1>(codes), fp4_decode2_f32<2>(codes),
                      fp4_decode2_f32<3>(codes)};
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = (__bf16)(q[j].x * e);
    r[2 * j + 1] = (__bf16)(q[j].y * e);
  }
  return r;
}

template <int OUT>
__device__ __forceinline__ void store_out(void *c, int64_t ldc, int64_t row, int64_t col, float v) {
  if (OUT == 0) static_cast<float *>(c)[row * ldc + col] = v;
  else static_cast<__bf16 *>(c)[row * ldc + col] = (__bf16)v;
}

// MODE 0 = W4A4 (fp16 MFMA), 1 = W4A16 (bf16 MFMA).  WM x WN waves of (BM/WM) x (BN/WN).
//
// LDS: a ring of three stages, the DMA two stages ahead of the MFMAs.  Stage layout:
//   A codes   [BM/32][2 parts][64 lanes][16 B]   (MODE 0)  or  A bf16 [BM/32][8 steps][64 lanes][16 B]
//   A scales  [BM/32][64 lanes][4 B]             (MODE 0)
//   B codes   [BN/32][2 parts][64 lanes][16 B]   B scales [BN/32 rounded up to 4][64 lanes][4 B]
// A stage is one 128-k chunk, except for W4A16 with half-chunk stages (HS)
// (part p: A bf16 [BM/32][4 steps][64 lanes][16 B], B codes [BN/32][64 lanes][16 B]).
// Each 1-KB (or 256-B) block is filled by one wave-wide LDS-DMA load whose lane addresses implement
// the row-major -> lane-order permutation for A; B is prepacked in exactly this order.  Rows past
// M and columns past N are clamped to the last valid one (their results are never stored).  The
// W4A4 loop and the two W4A16 loops below describe their own register pipelines.
// ABLK: values per A scale byte along K (16, 32 or 64; W4A4).  Lane l = r + 32 h needs the bytes of
// the blocks under its 64 k of a chunk: 4, 2 or 1 bytes, fetched as the aligned dword holding them
// and shifted into place when read.
// Two workgroups per CU (a grid a little larger than the CU count runs in one round, and one wave's
// VALU work runs beside the other's MFMAs): W4A4 128 x 128 and 128 x 192 tiles (64 / 96
// accumulators per wave) and W4A16 128 x 256 tiles with half-chunk stages (128); larger tiles one
// wave per SIMD.  (W4A16 64 x 256 tiles get the same register budget, but their three whole-chunk
// stages, 102 KB of LDS, leave room for one workgroup per CU.)
template <int MODE, int BM, int BN, int WM, int WN, int OUT, int ABLK, bool HS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    (BM * BN <= 128 * 192 || (HS && BM == 128)) ? 2 : 1, (BM * BN <= 128 * 192 || (HS && BM == 128)) ? 2 : 1))) void k_gemm_tiled(
    const void *__restrict__ a, const uint8_t *__restrict__ a_scales, const float *__restrict__ a_ts,
    const uint8_t *__restrict__ bp, const float *__restrict__ b_ts, int M, int N, int K, int64_t lda,
    void *__restrict__ c, int64_t ldc, int tiles_m, int tiles_n, int m_off, int n_off, int splits,
    float *__restrict__ partial, QuantOut qo) {
  using Cfg = TileCfg<MODE, BM, BN, HS>;
  constexpr int TM = BM / WM / 32;  // MFMA tiles per wave along M
  constexpr int TN = BN / WN / 32;
  constexpr bool HALF = Cfg::kHalf;
  constexpr int NA = (MODE == 0) ? (BM / 32) * 2 : (BM / 32) * (HALF ? 4 : 8);  // 1-KB A blocks per stage
  constexpr int NAS = (MODE == 0) ? BM / 32 : 0;                                 // 256-B A scale blocks
  constexpr int NB = (BN / 32) * (HALF ? 1 : 2), NBS = Cfg::kBSUnits;
  static_assert(NA % 4 == 0 && NB % 4 == 0 && NBS % 4 == 0 && NAS % 4 == 0, "block counts");
  static_assert(4 * 32 * EpiPitch<BN / WN, 4>::kPitch <= 3 * Cfg::kStage, "epilogue staging fits the LDS ring");
  constexpr int kAStep = (MODE == 0) ? 64 : 256;  // A bytes per row per chunk
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // XCD-aware tile order: consecutive dispatches land on different XCDs; give each XCD a
  // contiguous range of tiles in grouped-raster order (4 tile rows at a time) so its L2 sees
  // shared A rows and shared B columns.
  // Split-K: workgroup = (tile, split); split s covers chunks [s Kc / splits, (s+1) Kc / splits).
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int nwg = ntiles * splits;
    const int full = (nwg / 8) * 8;  // bijective remap on the multiple-of-8 prefix
    if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  }
  const int split = bid / ntiles;
  bid -= split * ntiles;
  int tile_m, tile_n;
  grouped_tile<4>(bid, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = m_off + tile_m * BM, n0 = n_off + tile_n * BN;

  const int Kc = K / kChunk;
  const int kbeg = (int)((int64_t)split * Kc / splits), kend = (int)((int64_t)(split + 1) * Kc / splits);
  const int Nu = (N + 31) / 32;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  const int lh = lane >> 5, lr = lane & 31;

  // ---- sources of this wave's LDS-DMA loads: wave-uniform bases (SGPRs) + 32-bit lane offsets ----
  // A rows past M are clamped to M - 1 and B units past N to the last unit (results never stored).
  // The host guarantees BM * (A row bytes) < 2^31, so the A lane offsets fit in 32 bits.
  const int64_t arow_bytes = (MODE == 0) ? lda / 2 : lda * 2;
  const uint8_t *a_tile = static_cast<const uint8_t *>(a) + (int64_t)m0 * arow_bytes;
  static_assert(ABLK == 16 || ABLK == 32 || ABLK == 64, "A block size");
  const uint8_t *as_tile = (MODE == 0) ? a_scales + (int64_t)m0 * (lda / ABLK) : nullptr;
  uint32_t oa[NA / 4];
  uint32_t oas[NAS / 4 > 0 ? NAS / 4 : 1];
#pragma unroll
  for (int i = 0; i < NA / 4; ++i) {
    const int q = wave + 4 * i;
    if (MODE == 0) {
      const int sub = q >> 1, part = q & 1;
      const int row = min(m0 + sub * 32 + lr, M - 1) - m0;
      oa[i] = (uint32_t)(row * (uint32_t)arow_bytes) + 32 * lh + 16 * part;
    } else {
      // lane (r, h) of step st holds A[row r][k = 64 h + 8 st .. + 8) of the chunk (as B's lanes);
      // a half-chunk stage holds steps 4 p .. 4 p + 3 of part p (its offset 64 p bytes added at issue)
      const int sub = HALF ? q >> 2 : q >> 3, st = HALF ? q & 3 : q & 7;
      const int row = min(m0 + sub * 32 + lr, M - 1) - m0;
      oa[i] = (uint32_t)(row * (uint32_t)arow_bytes) + 2 * (64 * lh + 8 * st);
    }
  }
#pragma unroll
  for (int i = 0; i < NAS / 4; ++i) {
    const int q = wave + 4 * i;
    const int row = min(m0 + q * 32 + lr, M - 1) - m0;
    // byte index (in the tile's scale rows) of the lane's first block in chunk 0: 16-blocks are
    // dword aligned (lda % 64 == 0), 32-blocks come as the row's dword per chunk (the lane's pair
    // is bytes 2h, 2h + 1), a 64-block's byte sits at a chunk-dependent position in its dword
    oas[i] = (uint32_t)(row * (uint32_t)(lda / ABLK)) + (ABLK == 16 ? 4 * lh : (ABLK == 64 ? lh : 0));
  }
  const uint32_t ob = lane * 16, obs = lane * 4;
  // prepacked B unit (n-unit nu, chunk kc) of this wave's q-th block
  auto b_unit = [&](int q, int kc) -> uint64_t {
    const int nu = min(n0 / 32 + q, Nu - 1);
    return ((uint64_t)nu * (uint64_t)Kc + (uint64_t)kc);
  };

  // kc: the chunk; HALF: kc is the half-chunk stage g (chunk g / 2, part g % 2)
  auto issue_slot = [&](int kc, int buf, int t) {
    uint8_t *st = smem + buf * Cfg::kStage;
    const int part = HALF ? (kc & 1) : 0;
    if (HALF) kc >>= 1;
    if (t < NA / 4) {
      g2l16(a_tile + (int64_t)kc * kAStep + 64 * part + oa[t], st + (wave + 4 * t) * 1024);
    } else if (t < NA / 4 + NAS / 4) {
      const int i = t - NA / 4;
      if constexpr (ABLK == 64)
        g2l4(as_tile + ((oas[i] + 2u * (uint32_t)kc) & ~3u), st + Cfg::kALds + (wave + 4 * i) * 256);
      else
        g2l4(as_tile + kc * (128 / ABLK) + oas[i], st + Cfg::kALds + (wave + 4 * i) * 256);
    } else if (t < NA / 4 + NAS / 4 + NB / 4) {
      const int i = t - NA / 4 - NAS / 4, q = wave + 4 * i;
      if (HALF)
        g2l16(bp + b_unit(q, kc) * 2048ull + part * 1024 + ob, st + Cfg::kALds + Cfg::kASLds + q * 1024);
      else
        g2l16(bp + b_unit(q >> 1, kc) * 2048ull + (q & 1) * 1024 + ob, st + Cfg::kALds + Cfg::kASLds + q * 1024);
    } else {
      const int i = t - NA / 4 - NAS / 4 - NB / 4, q = wave + 4 * i;
      g2l4(bp + scale_region + b_unit(q, kc) * 256ull + obs, st + Cfg::kALds + Cfg::kASLds + Cfg::kBLds + q * 256);
    }
  };
  constexpr int NSLOT = NA / 4 + NAS / 4 + NB / 4 + NBS / 4;
  auto issue = [&](int kc, int buf) {
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) issue_slot(kc, buf, t);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (kend <= kbeg) {
    // empty K range (not produced by the planner): leave the accumulators at zero
  } else if (MODE == 0) {
    // ---- W4A4: one continuous stream of 16-k steps.  Dequantization is a two-stage pipeline that
    // runs beside step s's 16 MFMAs (also across chunk boundaries): the codes of step s+2 are
    // decoded to exact E2M1 values (Q registers) and the decoded values of step s+1 are multiplied
    // by their block scales (F registers), so no VALU result is consumed by the next instruction
    // and the VALU work co-issues with the MFMAs.  Codes are held per half-chunk ("part", 4 steps):
    // part 1 of chunk kc is read at the start of chunk kc, part 0 of chunk kc+1 (and its scales) at
    // step 3, so every LDS read has >= 3 steps of MFMA work to land.  A 3-stage LDS ring with the
    // DMA two chunks ahead leaves one barrier per chunk.
    u32x4 P0a[TM], P0b[TN], P1a[TM], P1b[TN];
    uint32_t Sa[TM], Sb[TN];
    f16x2 Ea[TM][2], Eb[TN][2], Na[TM][2], Nb[TN][2];
    f16x8 Fa[2][TM], Fb[2][TN], Qa[2][TM], Qb[2][TN];

    auto stage = [&](int buf) { return smem + buf * Cfg::kStage; };
    auto read_part = [&](u32x4 *ra, u32x4 *rb, int buf, int part) {
      const uint8_t *st = stage(buf);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int sub = wm * (BM / WM / 32) + i;
        ra[i] = *reinterpret_cast<const u32x4 *>(st + ((sub * 2 + part) * 64 + lane) * 16);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int unit = wn * (BN / WN / 32) + j;
        rb[j] = *reinterpret_cast<const u32x4 *>(st + Cfg::kALds + Cfg::kASLds + ((unit * 2 + part) * 64 + lane) * 16);
      }
    };
    // kabs: the absolute chunk whose data the stage holds (it fixes a 64-block's byte position)
    auto read_scales = [&](int buf, int kabs) {
      const uint8_t *st = stage(buf);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int sub = wm * (BM / WM / 32) + i;
        const uint32_t w = *reinterpret_cast<const uint32_t *>(st + Cfg::kALds + (sub * 64 + lane) * 4);
        if constexpr (ABLK == 16) {
          Sa[i] = w;
        } else if constexpr (ABLK == 32) {
          Sa[i] = w >> (16 * lh);
        } else {
          // the byte position of the row being read (this wave's sub-tile, not the rows this wave
          // fetched), exactly as the fetch computed it
          const uint32_t row = (uint32_t)(min(m0 + sub * 32 + lr, M - 1) - m0);
          Sa[i] = w >> (8 * ((row * (uint32_t)(lda / ABLK) + lh + 2u * (uint32_t)kabs) & 3u));
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int unit = wn * (BN / WN / 32) + j;
        const uint32_t w = *reinterpret_cast<const uint32_t *>(st + Cfg::kALds + Cfg::kASLds + Cfg::kBLds + (unit * 64 + lane) * 4);
        Sb[j] = w;
      }
    };
    auto cvt_scales = [&](f16x2 (*ea)[2], f16x2 (*eb)[2]) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ea[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(Sa[i], 1.0f, false);
        ea[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(Sa[i], 1.0f, true);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // units past N hold a clamped copy of the last unit and their results are never stored:
        // zero scales make their operands zero, which draws less power in the matrix cores
        const uint32_t sb = (n0 / 32 + wn * (BN / WN / 32) + j < Nu) ? Sb[j] : 0u;
        eb[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
        eb[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, true);
      }
    };
    // stage 1: decode the codes of step s (0..7) of a chunk from part registers (ra, rb) into Q[s & 1]
    auto cvt_step = [&](const u32x4 *ra, const u32x4 *rb, int s) {
      const int q = s & 3, slot = s & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) Qa[slot][i] = decode_f16x8(ra[i][q]);
#pragma unroll
      for (int j = 0; j < TN; ++j) Qb[slot][j] = decode_f16x8(rb[j][q]);
    };
    // stage 2: F[s & 1] = Q[s & 1] * block scale of step s, with scales (ea, eb) of its chunk
    auto mul_step = [&](f16x2 (*ea)[2], f16x2 (*eb)[2], int s) {
      const int blk = s >> 1, slot = s & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        // the lane's byte for step s: 16-blocks: s / 2 of 4; 32-blocks: s / 4 of 2; 64: the one
        const _Float16 e = (ABLK == 16) ? ea[i][blk >> 1][blk & 1] : (ABLK == 32 ? ea[i][0][s >> 2] : ea[i][0][0]);
        Fa[slot][i] = scale_f16x8(Qa[slot][i], e);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) Fb[slot][j] = scale_f16x8(Qb[slot][j], eb[j][blk >> 1][blk & 1]);
    };
    auto mfma_step = [&](int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Fb[slot][j], Fa[slot][i], acc[i][j], 0, 0, 0);
    };
    auto interleave = [&]() {
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, (8 * (TM + TN)) / (TM * TN) + 1, 0);  // VALU
      }
    };

    // Prologue: start on chunk 0 as soon as it has landed; chunk 1 keeps streaming and is waited
    // for in the first chunk's step 3, right before its first LDS read.
    constexpr int kPer = (NSLOT + 5) / 6;                                 // DMA loads per step
    constexpr int kIssuedBefore3 = (3 * kPer < NSLOT) ? 3 * kPer : NSLOT;  // issued in steps 0-2
    const int nk = kend - kbeg;
    issue(kbeg, 0);
    if (nk > 1) {
      issue(kbeg + 1, 1);
      wait_vmem_then_barrier<NSLOT>();  // this wave's chunk-0 loads (chunk 1's may be in flight)
    } else {
      wait_vmem_then_barrier<0>();
    }
    read_part(P0a, P0b, 0, 0);
    read_scales(0, kbeg);
    cvt_scales(Ea, Eb);
    cvt_step(P0a, P0b, 0);
    cvt_step(P0a, P0b, 1);
    mul_step(Ea, Eb, 0);
    __builtin_amdgcn_sched_barrier(0);

    // One chunk of 8 steps.  FIRST (compile time) is the peeled first chunk: it has no top wait
    // but waits for chunk 1 before step 3; later chunks wait for the next chunk at the top.
    auto chunk = [&](int kc, auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      const int cur = kc % 3;
      if (!FIRST) {
        wait_vmem();  // this wave's DMA of chunk kc+1 (issued one chunk ago) has landed
        __syncthreads();
      }
      // Branch-free steps (a branch would split the scheduling region): near the end of K the
      // DMA re-fetches the last chunk into the free stage and the look-ahead reads/dequantizes a
      // stale stage; neither result is used.
      const int kdma = kbeg + min(kc + 2, nk - 1);
      const int bdma = (kc + 2) % 3, bnext = (kc + 1) % 3;
      read_part(P1a, P1b, cur, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int slot = s & 1;
        if (FIRST && s == 3) {
          // chunk 1 (issued in the prologue, before this chunk's DMA) must have landed everywhere
          if (nk > 1) wait_vmem_then_barrier<kIssuedBefore3>();
          __builtin_amdgcn_sched_barrier(0);
        }
        // spread chunk kc+2's DMA over the steps: a VMEM issue stall then overlaps running MFMAs
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if (s * kPer + u < NSLOT) issue_slot(kdma, bdma, s * kPer + u);
        if (s == 3) {
          read_part(P0a, P0b, bnext, 0);  // P0 of this chunk was last decoded in step 1
          read_scales(bnext, kbeg + min(kc + 1, nk - 1));
        }
        if (s == 6) cvt_scales(Na, Nb);
        // stage 2 for step s+1, stage 1 for step s+2 (steps 8 and 9 are the next chunk's 0 and 1)
        if (s < 7) mul_step(Ea, Eb, s + 1);
        else mul_step(Na, Nb, 0);
        if (s < 2) cvt_step(P0a, P0b, s + 2);
        else if (s < 6) cvt_step(P1a, P1b, s + 2);
        else cvt_step(P0a, P0b, s - 6);
        mfma_step(slot);
        interleave();
        if (s < 6) __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);  // this step's DMA loads
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) { Ea[i][0] = Na[i][0]; Ea[i][1] = Na[i][1]; }
#pragma unroll
      for (int j = 0; j < TN; ++j) { Eb[j][0] = Nb[j][0]; Eb[j][1] = Nb[j][1]; }
    };
    chunk(0, std::true_type{});
    for (int kc = 1; kc < nk; ++kc) chunk(kc, std::false_type{});
  } else if constexpr (HALF) {
    // ---- W4A16, half-chunk stages (part p of each chunk: its 4 MFMA steps); per stage the wave's
    // B codes and scales into registers, the DMA of stage g + 2 into the third buffer, then 4 steps
    // with the next step's B dequantization and A reads pipelined beside the current step's MFMAs.
    // Each dequantized B fragment feeds TM = 4 MFMAs. ----
    const int ng = 2 * (kend - kbeg);
    issue(2 * kbeg, 0);
    if (ng > 1) {
      issue(2 * kbeg + 1, 1);
      wait_vmem_then_barrier<NSLOT>();
    } else {
      wait_vmem_then_barrier<0>();
    }
    for (int g = 0; g < ng; ++g) {
      const int cur = g % 3;
      if (g > 0) {
        if (g + 1 < ng) wait_vmem_then_barrier<NSLOT>();  // stage g + 1's DMA may be outstanding
        else wait_vmem_then_barrier<0>();
      }
      const uint8_t *st = smem + cur * Cfg::kStage;
      const uint8_t *sA = st, *sB = st + Cfg::kALds, *sBS = sB + Cfg::kBLds;
      u32x4 bc[TN];
      uint32_t bsw[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int unit = wn * (BN / WN / 32) + j;
        bsw[j] = *reinterpret_cast<const uint32_t *>(sBS + (unit * 64 + lane) * 4);
        bc[j] = *reinterpret_cast<const u32x4 *>(sB + (unit * 64 + lane) * 16);
      }
      if (g + 2 < ng) issue(2 * kbeg + g + 2, (g + 2) % 3);
      // part p's steps 4 p + q use the lane's 16-k blocks 2 p + q / 2 (scale bytes 2 p, 2 p + 1)
      const int p = g & 1;
      float eb[TN][2];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) eb[j][t] = e4m3_to_f32((bsw[j] >> (16 * p + 8 * t)) & 0xffu);
      bf16x8 bf[2][TN];
      u32x4 ar[2][TM];
      auto deq = [&](int q, int slot) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[slot][j] = dequant_bf16x8(bc[j][q], eb[j][q >> 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int sub = wm * (BM / WM / 32) + i;
          ar[slot][i] = *reinterpret_cast<const u32x4 *>(sA + ((sub * 4 + q) * 64 + lane) * 16);
        }
      };
      deq(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int slot = q & 1;
        if (q + 1 < 4) deq(q + 1, slot ^ 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const bf16x8 afr = __builtin_bit_cast(bf16x8, ar[slot][i]);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[slot][j], afr, acc[i][j], 0, 0, 0);
        }
        if (q + 1 < 4) {
#pragma unroll
          for (int t = 0; t < TM * TN; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (18 * TN) / (TM * TN) + 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // ---- W4A16: chunk fragments into registers, next chunk's DMA, 8 pipelined steps ----
    // The DMA of chunk kc + 2 is issued during chunk kc into the third stage; a chunk waits only for
    // its own DMA (the next chunk's may still be in flight), so the loads have two chunks to land.
    const int nk = kend - kbeg;
    issue(kbeg, 0);
    if (nk > 1) {
      issue(kbeg + 1, 1);
      wait_vmem_then_barrier<NSLOT>();
    } else {
      wait_vmem_then_barrier<0>();
    }
    for (int kc = 0; kc < nk; ++kc) {
      const int cur = kc % 3;
      if (kc > 0) {
        if (kc + 1 < nk) wait_vmem_then_barrier<NSLOT>();  // chunk kc + 1's DMA may be outstanding
        else wait_vmem_then_barrier<0>();                 // nothing was issued after chunk kc
      }
      const uint8_t *st = smem + cur * Cfg::kStage;
      const uint8_t *sA = st, *sB = st + Cfg::kALds + Cfg::kASLds, *sBS = sB + Cfg::kBLds;
      u32x4 bc[2][TN];
      uint32_t bsw[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int unit = wn * (BN / WN / 32) + j;
        bsw[j] = *reinterpret_cast<const uint32_t *>(sBS + (unit * 64 + lane) * 4);
#pragma unroll
        for (int p = 0; p < 2; ++p) bc[p][j] = *reinterpret_cast<const u32x4 *>(sB + ((unit * 2 + p) * 64 + lane) * 16);
      }
      if (kc + 2 < nk) issue(kbeg + kc + 2, (kc + 2) % 3);
      float eb[TN][4];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) eb[j][t] = e4m3_to_f32((bsw[j] >> (8 * t)) & 0xffu);
      bf16x8 bf[2][TN];
      u32x4 ar[2][TM];
      auto read_a = [&](int s, int slot) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int sub = wm * (BM / WM / 32) + i;
          ar[slot][i] = *reinterpret_cast<const u32x4 *>(sA + ((sub * 8 + s) * 64 + lane) * 16);
        }
      };
      auto deq_b = [&](int s, int slot) {
        const int p = s >> 2, q = s & 3, blk = s >> 1;
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[slot][j] = dequant_bf16x8(bc[p][j][q], eb[j][blk]);
      };
      read_a(0, 0);
      deq_b(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int slot = s & 1;
        // The next step's A reads go out before this step's MFMAs, which hide their latency.  The
        // wait for this step's reads (issued a step ago) is explicit and comes first: left to the
        // compiler, the wait in front of the MFMAs would also cover the reads just issued.
        if (s + 1 < 8) {
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
          read_a(s + 1, slot ^ 1);
          __builtin_amdgcn_sched_barrier(0);
          deq_b(s + 1, slot ^ 1);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const bf16x8 afr = __builtin_bit_cast(bf16x8, ar[slot][i]);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[slot][j], afr, acc[i][j], 0, 0, 0);
        }
        if (s + 1 < 8) {
#pragma unroll
          for (int t = 0; t < TM * TN; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (18 * TN) / (TM * TN) + 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: scale by S_A * S_B, convert, store ---------------------------------------------
  wait_vmem();      // the loop's last look-ahead DMA targets the ring, which now stages output
  __syncthreads();  // every wave is done reading the LDS ring
  uint8_t *lds_wave = smem + wave * (32 * EpiPitch<BN / WN, 4>::kPitch);
  const int row0 = m0 + wm * (BM / WM), col0 = n0 + wn * (BN / WN);
  if (splits > 1) {
    // unscaled fp32 partial tile -> partial[split][M][N]; the reduce kernel scales and converts
    const bool vec = (N % 4 == 0);  // 16-byte aligned rows; lanes check their own bounds
    store_tile<BN / WN, TM, TN, float, kPartialNT>(acc, 1.0f, partial + (int64_t)split * M * N, N, M, N, row0, col0,
                                                   vec, lds_wave, lane);
    return;
  }
  const float sab = (MODE == 0) ? (*a_ts) * (*b_ts) : *b_ts;
  if constexpr (OUT == 2) {
    store_tile_nvfp4<BN / WN, TM, TN>(acc, sab, qo, M, N, row0, col0, lds_wave, lane);
  } else {
    typedef typename std::conditional<OUT == 0, float, __bf16>::type OutT;
    const bool vec = (ldc * (int64_t)sizeof(OutT)) % 16 == 0;  // 16-byte aligned rows
    store_tile<BN / WN, TM, TN, OutT, kOutputNT>(acc, sab, static_cast<OutT *>(c), ldc, M, N, row0, col0, vec,
                                                 lds_wave, lane);
  }
}

// ---- generic fallback (any K % 16 == 0): one thread per output element ---------------------------

__device__ __forceinline__ float prepacked_weight(const uint8_t *bp, int64_t Kc, uint64_t scale_region, int64_t n,
                                                  int64_t k) {
  const int64_t nu = n >> 5, kc = k >> 7, kk = k & 127;
  const int h = (int)(kk >> 6), lane = (int)(n & 31) + 32 * h;
  const int in_lane = (int)(kk & 63);  // code index within the lane's 64
  const int part = in_lane >> 5, byte = (in_lane & 31) >> 1;
  const uint64_t unit = (uint64_t)nu * (uint64_t)Kc + (uint64_t)kc;
  const uint8_t cb = bp[unit * 2048 + (uint64_t)part * 1024 + (uint64_t)lane * 16 + byte];
  const uint32_t code = (in_lane & 1) ? (cb >> 4) : (cb & 15u);
  const uint8_t sb = bp[scale_region + unit * 256 + (uint64_t)lane * 4 + ((in_lane >> 4) & 3)];
  const f32x2 q = fp4_decode2_f32<0>(code);
  return q.x * e4m3_to_f32(sb);
}

template <int MODE, int OUT>
__global__ __launch_bounds__(256) void k_gemm_generic(const void *__restrict__ a, const uint8_t *__restrict__ a_scales,
                                                      const float *__restrict__ a_ts, const uint8_t *__restrict__ bp,
                                                      const float *__restrict__ b_ts, int64_t M, int64_t N, int64_t K,
                                                      int64_t lda, int ablk, void *__restrict__ c, int64_t ldc) {
  const int64_t Kc = (K + 127) / 128, Nu = (N + 31) / 32;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  const float sab = (MODE == 0) ? (*a_ts) * (*b_ts) : *b_ts;
  for (int64_t t = blockIdx.x * 256ll + threadIdx.x; t < M * N; t += (int64_t)gridDim.x * 256) {
    const int64_t n = t % N, m = t / N;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float av;
      if (MODE == 0) {
        const uint8_t cb = static_cast<const uint8_t *>(a)[m * (lda / 2) + (k >> 1)];
        const uint32_t code = (k & 1) ? (cb >> 4) : (cb & 15u);
        const f32x2 q = fp4_decode2_f32<0>(code);
        av = q.x * e4m3_to_f32(a_scales[m * (lda / ablk) + k / ablk]);
      } else {
        av = __uint_as_float((uint32_t) static_cast<const uint16_t *>(a)[m * lda + k] << 16);
      }
      acc = fmaf(av, prepacked_weight(bp, Kc, scale_region, n, k), acc);
    }
    store_out<OUT>(c, ldc, m, n, acc * sab);
  }
}

// ---- split-K reduction: C = (sum over splits, in order) * S_A S_B, deterministic ----------------
// OUT 2 writes NVFP4 (QuantOut): a thread sums and requantizes one 16-value block.

template <int OUT>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ partial, int splits, int M, int N,
                                                       void *__restrict__ c, int64_t ldc, const float *__restrict__ a_ts,
                                                       const float *__restrict__ b_ts, QuantOut qo) {
  const float sab = (a_ts ? *a_ts : 1.0f) * (b_ts ? *b_ts : 1.0f);
  const int64_t MN = (int64_t)M * N;
  if constexpr (OUT == 2) {
    // a thread owns one 16-value block (N % 16 == 0)
    const QuantConsts qc = make_quant_consts(*qo.out_ts, false);
    for (int64_t b = blockIdx.x * 256ll + threadIdx.x; b < MN / 16; b += (int64_t)gridDim.x * 256) {
      float v[16];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(partial + 16 * b + 4 * h);
        for (int sp = 1; sp < splits; ++sp) a += *reinterpret_cast<const f32x4 *>(partial + sp * MN + 16 * b + 4 * h);
        a *= sab;
        v[4 * h] = a.x;
        v[4 * h + 1] = a.y;
        v[4 * h + 2] = a.z;
        v[4 * h + 3] = a.w;
      }
      requant16(v, (16 * b) / N, (16 * b) % N, true, N, qo, qc);
    }
    return;
  }
  const bool vec = (ldc % 4 == 0);  // 4-element stores stay aligned (c is 16-byte aligned)
  const int64_t nq = MN / 4;  // N % 4 == 0 here
  for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < nq; q += (int64_t)gridDim.x * 256) {
    f32x4 acc = __builtin_bit_cast(f32x4, load16<kReduceNT>(partial + 4 * q));
    for (int sp = 1; sp < splits; ++sp) acc += __builtin_bit_cast(f32x4, load16<kReduceNT>(partial + sp * MN + 4 * q));
    const int64_t m = (4 * q) / N, n = (4 * q) % N;
    acc *= sab;
    if (OUT == 0) {
      float *dst = static_cast<float *>(c) + m * ldc + n;
      if (vec) {
        store16<kOutputNT>(dst, __builtin_bit_cast(u32x4, acc));
      } else {
        dst[0] = acc.x;
        dst[1] = acc.y;
        dst[2] = acc.z;
        dst[3] = acc.w;
      }
    } else {
      __bf16 *dst = static_cast<__bf16 *>(c) + m * ldc + n;
      if (vec) {
        const bf16x2 h0 = {(__bf16)acc.x, (__bf16)acc.y}, h1 = {(__bf16)acc.z, (__bf16)acc.w};
        u32x2 o;
        o.x = __builtin_bit_cast(uint32_t, h0);
        o.y = __builtin_bit_cast(uint32_t, h1);
        if constexpr (kOutputNT) __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(dst));
        else *reinterpret_cast<u32x2 *>(dst) = o;
      } else {
        dst[0] = (__bf16)acc.x;
        dst[1] = (__bf16)acc.y;
        dst[2] = (__bf16)acc.z;
        dst[3] = (__bf16)acc.w;
      }
    }
  }
}

hipError_t launch_splitk_reduce(const float *partial, int splits, int64_t M, int64_t N, void *c, int out_dtype,
                                int64_t ldc, const float *a_ts, const float *b_ts, const QuantOut &qo,
                                hipStream_t stream) {
  int64_t grid = (M * N / (out_dtype == 2 ? 16 : 4) + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  if (out_dtype == 0)
    k_splitk_reduce<0><<<(unsigned)grid, 256, 0, stream>>>(partial, splits, (int)M, (int)N, c, ldc, a_ts, b_ts, qo);
  else if (out_dtype == 1)
    k_splitk_reduce<1><<<(unsigned)grid, 256, 0, stream>>>(partial, splits, (int)M, (int)N, c, ldc, a_ts, b_ts, qo);
  else
    k_splitk_reduce<2><<<(unsigned)grid, 256, 0, stream>>>(partial, splits, (int)M, (int)N, c, ldc, a_ts, b_ts, qo);
  return hipGetLastError();
}

// ---- launchers ----------------------------------------------------------------------------------

template <int MODE, int BM, int BN, int WM, int WN, int OUT, int ABLK = 16, bool HS = false>
static hipError_t launch_tiled(const GemmArgs &g, int m_off, int n_off, int m_len, int n_len, int splits,
                               float *partial, hipStream_t stream) {
  using Cfg = TileCfg<MODE, BM, BN, HS>;
  const int tm = (m_len + BM - 1) / BM, tn = (n_len + BN - 1) / BN;
  auto kern = k_gemm_tiled<MODE, BM, BN, WM, WN, OUT, ABLK, HS>;
  const int smem = 3 * Cfg::kStage;
  static std::atomic<bool> configured[kMaxDevices];  // per instantiation and device
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), smem, configured);
  if (e != hipSuccess) return e;
  kern<<<tm * tn * splits, 256, smem, stream>>>(g.a, g.a_scales, g.a_ts, static_cast<const uint8_t *>(g.b), g.b_ts,
                                                (int)g.M, (int)g.N, (int)g.K, g.lda, g.c, g.ldc, tm, tn, m_off, n_off,
                                                splits, partial, g.qo);
  return hipGetLastError();
}

template <int MODE, int OUT>
static hipError_t launch_generic(const GemmArgs &g, hipStream_t stream) {
  int64_t total = g.M * g.N;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  k_gemm_generic<MODE, OUT><<<(unsigned)grid, 256, 0, stream>>>(g.a, g.a_scales, g.a_ts,
                                                                 static_cast<const uint8_t *>(g.b), g.b_ts, g.M, g.N,
                                                                 g.K, g.lda, g.a_blk, g.c, g.ldc);
  return hipGetLastError();
}

// Plan: which tile kernel(s) (W4A4: 256x256, 128x192 or 128x128; W4A16: 128x256 with whole- or
// half-chunk stages, 64x256, or the skinny kernel), how many K splits, and an optional split of N
// into a region of 256x256 tiles (exactly one round on the chip) plus a remainder of 128x128 tiles.
GemmPlan plan_gemm(int mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  GemmPlan pl;
  const int64_t arow_bytes = (mode == 0) ? lda / 2 : lda * 2;
  if (K % kChunk != 0 || (mode == 0 && lda % kChunk != 0) || 256 * arow_bytes >= (int64_t(1) << 31)) {
    // the tiled kernels need whole 128-k chunks and 32-bit A offsets within a 256-row tile
    pl.variant = GemmVariant::Generic;
    return pl;
  }
  const int64_t cus = 256;  // planning for the MI355X chip (256 CUs)
  const int64_t Kc = K / kChunk;
  if (mode == 1) {
    const int64_t Nu = (N + 31) / 32;
    if (M <= kSkinnyMaxM && 32 * lda < (int64_t(1) << 31)) {
      // streaming: narrow N splits K across workgroups (each split keeps >= 16 chunks), doubling
      // the splits while the doubled grid stays under 1.5 workgroups per CU (N 3072, K 12288:
      // two splits, 10.9 us at M = 1 against 11.7 us with four); waves per workgroup grow with
      // the chunks per split
      pl.variant = GemmVariant::W4A16_Skinny;
      int64_t sp = 1;
      while (2 * Nu * sp < (3 * cus) / 2 && Kc / (2 * sp) >= 16 && N % 4 == 0) sp *= 2;
      pl.splits = (int)sp;
      const int64_t per = Kc / sp;
      pl.waves = per >= 48 ? 16 : (per >= 16 ? 8 : 4);
      return pl;
    }
    // Tiles of 128 x 256 with whole-chunk stages (one workgroup per CU) or half-chunk stages (two
    // workgroups per CU: one wave's dequantization runs beside the other's MFMAs), or of 64 x 256
    // (twice the dequantization per MFMA, but twice the workgroups before K has to be split), and a
    // K split, by a cost model fit to measurements (M 64..4096, N and K 1024..12288; the two-per-CU
    // form on a sweep of 30 shapes, M 128..4096, and the 64-row form on 30 more, M 96..768, over
    // five N x K pairs): chunks per split x a chunk's time for the form and the workgroups a CU runs
    // (whole-chunk 128 x 256: 1.99 us per workgroup, one at a time; half-chunk: 3.5 us for two
    // sharing a CU, 2.2 us for one alone; 64 x 256: 1.5 us, one at a time), plus, for a split, the
    // fp32 partials' traffic (written, read back, output written) and the reduction's launch.
    // Splits keep >= 6 chunks each.  Against the one-per-CU forms alone: up projection N 12288, K
    // 3072 at M = 256 43 -> 40 us, 1024 103 -> 82 us, 4096 308 -> 268 us; down (N 3072, K 12288)
    // at M = 4096 331 -> 300 us; N 1024 / 4096 / 8192 at M <= 512 by 10-27 %.  (256 x 256 tiles,
    // one per CU at 3.71 us a chunk, were slower than the two-per-CU form on every shape measured.)
    double best_t = 1e300;
    for (int form = 0; form < 3; ++form) {
      const int64_t bm = form == 2 ? 64 : 128;
      const int64_t tiles = ((M + bm - 1) / bm) * ((N + 255) / 256);
      for (int sp = 1; sp <= 16; ++sp) {
        if (sp > 1 && (Kc / sp < 6 || N % 4 != 0)) continue;
        const int64_t per_cu = (tiles * sp + cus - 1) / cus;  // workgroups per CU, rounded up
        const double chunks = (double)((Kc + sp - 1) / sp);
        double t = form == 1 ? chunks * ((double)(per_cu / 2) * 3.5 + (double)(per_cu % 2) * 2.2)
                             : chunks * (double)per_cu * (form == 2 ? 1.5 : 1.99);
        if (sp > 1) t += (8.0 * sp + 2.0) * (double)M * (double)N / 5.19e6 + 3.0;
        if (t < best_t) {
          best_t = t;
          pl.variant = form == 0 ? GemmVariant::W4A16_128x256
                                 : (form == 1 ? GemmVariant::W4A16_128x256h : GemmVariant::W4A16_64x256);
          pl.splits = sp;
        }
      }
    }
    return pl;
  }
  const int64_t tmb = (M + 255) / 256, tnb = (N + 255) / 256, tb = tmb * tnb;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  // 128 x 192 tiles (two workgroups per CU at most): where 128 x 128 tiles put two workgroups on
  // some CUs and 128 x 192 tiles need fewer workgroups per CU, and 256 x 256 tiles would either fit
  // one round (then only when 128 x 192 takes at most two per CU) or need a second round.  A lone
  // 128 x 192 workgroup runs a chunk in ~1.34 us, two on a CU in ~2.5 us, against 0.9 / 1.53 us
  // for 128 x 128 and 2.9 us for 256 x 256 (one per CU), and there is no K split: PixArt proj
  // 4096 x 1152 x 1152 22.0 -> 18.3 us, fc2 4096 x 1152 x 4608 62.5 -> 54.5 us (no fp32 partials),
  // fc1 4096 x 4608 x 1152 57.7 -> 46.8 us (one launch instead of 256 x 256 plus 128 x 128 tiles);
  // qkv 4096 x 3456 x 1152 stays on 256 x 256 (39.6 against 42.5 us) -- one machine, 40 shapes
  // M 300..8192, N 768..4608, K 1152 / 4608, all consistent with this rule.
  const int64_t t192 = ((M + 127) / 128) * ((N + 191) / 192);
  const int64_t w128 = (t128 + cus - 1) / cus, w192 = (t192 + cus - 1) / cus;
  if (t128 > cus && w192 < w128 && (w192 <= 2 || (tb > cus && w192 <= 3))) {
    pl.variant = GemmVariant::W4A4_128x192;
    return pl;
  }
  pl.variant = GemmVariant::W4A4_256x256;
  if (tb >= cus) {
    // more than one round: cover whole big-tile rounds, finish the rest with 128x128 tiles
    const int64_t cols = cus / tmb;  // big-tile columns that make exactly one round
    if (cols >= 1 && cols < tnb && N % 128 == 0) {
      const int64_t rest = ((M + 127) / 128) * ((N - cols * 256 + 127) / 128);  // 128x128 remainder tiles
      if (rest <= cus) pl.n_big = cols * 256;
    }
    return pl;
  }
  // Fewer big tiles than CUs.  128x128 tiles run two workgroups per CU: when their grid fits one
  // round (<= one per CU, or close to two per CU everywhere, or K short enough that the uneven
  // share costs little) they beat splitting K over 256x256 tiles, whose partials cost HBM traffic
  // and a reduction.
  if (t128 <= cus) {
    // At most one 128x128 tile per CU: splitting K over the idle CUs pays when the chunks saved
    // outweigh the fp32 partials and the reduction launch.  Cost model fit to a sweep (M 256 ..
    // 1024, N 1152 / 3072, K 1152 .. 4608, splits 1 .. 6; it picks the fastest split or one
    // within 1 us on all 15 shapes): chunks per split x 0.9 us (x 1.7 where two workgroups share
    // a CU), plus 2 us + splits x M N x 8 B at 2.9 TB/s for a split (256 x 1152 x 1152: 12.1 ->
    // 10.8 us; 256 x 3072 x 4608: 37.3 -> 22.9 us).
    pl.variant = GemmVariant::W4A4_128x128;
    pl.splits = 1;
    if (N % 4 == 0) {
      double best = 0.9 * (double)Kc;
      for (int sp = 2; sp <= 6; ++sp) {
        if (Kc / sp < 2 || t128 * sp > 2 * cus) continue;
        const double t = 0.9 * (double)((Kc + sp - 1) / sp) * (t128 * sp > cus ? 1.7 : 1.0) + 2.0 +
                         (double)sp * (double)M * (double)N * 8.0 / 2.9e6;
        if (t < best) {
          best = t;
          pl.splits = sp;
        }
      }
    }
    return pl;
  }
  if (t128 <= 2 * cus && (t128 % cus == 0 || t128 % cus >= (3 * cus) / 4 || Kc <= 12)) {
    pl.variant = GemmVariant::W4A4_128x128;
    return pl;
  }
  // otherwise 256x256 tiles, splitting K over idle CUs when every split keeps >= 8 chunks
  int best = 1;
  for (int sp = 2; sp <= 4; ++sp)
    if (tb * sp <= cus && Kc / sp >= 8 && N % 4 == 0) best = sp;
  if (tb * 2 > cus) best = 1;  // already more than half the chip: a reduction costs more than it saves
  pl.splits = best;
  return pl;
}

size_t gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  const GemmPlan pl = plan_gemm(mode, M, N, K, lda);
  return pl.splits > 1 ? (size_t)pl.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

size_t gemm_requant_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  const GemmPlan pl = plan_gemm(mode, M, N, K, lda);
  const size_t mn = (size_t)M * (size_t)N * sizeof(float);
  // the generic and skinny kernels produce fp32 first; the reduction pass requantizes
  if (pl.variant == GemmVariant::Generic || pl.variant == GemmVariant::W4A16_Skinny) return (size_t)pl.splits * mn;
  return pl.splits > 1 ? (size_t)pl.splits * mn : 0;
}

template <int OUT, int ABLK>
static hipError_t run_plan(const GemmArgs &g, const GemmPlan &pl, hipStream_t stream) {
  const int M = (int)g.M, N = (int)g.N;
  switch (pl.variant) {
    case GemmVariant::W4A4_256x256: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<0, 256, 256, 2, 2, OUT, ABLK>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, g.a_ts, g.b_ts, g.qo, stream);
      }
      if (pl.n_big > 0 && pl.n_big < N) {
        hipError_t e = launch_tiled<0, 256, 256, 2, 2, OUT, ABLK>(g, 0, 0, M, (int)pl.n_big, 1, nullptr, stream);
        if (e != hipSuccess) return e;
        return launch_tiled<0, 128, 128, 2, 2, OUT, ABLK>(g, 0, (int)pl.n_big, M, N - (int)pl.n_big, 1, nullptr, stream);
      }
      return launch_tiled<0, 256, 256, 2, 2, OUT, ABLK>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A4_128x192: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<0, 128, 192, 2, 2, OUT, ABLK>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, g.a_ts, g.b_ts, g.qo, stream);
      }
      return launch_tiled<0, 128, 192, 2, 2, OUT, ABLK>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A4_128x128: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<0, 128, 128, 2, 2, OUT, ABLK>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, g.a_ts, g.b_ts, g.qo, stream);
      }
      return launch_tiled<0, 128, 128, 2, 2, OUT, ABLK>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A16_128x256: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<1, 128, 256, 1, 4, OUT>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, nullptr, g.b_ts, g.qo, stream);
      }
      return launch_tiled<1, 128, 256, 1, 4, OUT>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A16_64x256: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<1, 64, 256, 1, 4, OUT>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, nullptr, g.b_ts, g.qo, stream);
      }
      return launch_tiled<1, 64, 256, 1, 4, OUT>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A16_128x256h: {
      if (pl.splits > 1) {
        float *part = static_cast<float *>(g.workspace);
        hipError_t e = launch_tiled<1, 128, 256, 1, 4, OUT, 16, true>(g, 0, 0, M, N, pl.splits, part, stream);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, pl.splits, M, N, g.c, OUT, g.ldc, nullptr, g.b_ts, g.qo, stream);
      }
      return launch_tiled<1, 128, 256, 1, 4, OUT, 16, true>(g, 0, 0, M, N, 1, nullptr, stream);
    }
    case GemmVariant::W4A16_Skinny:
      return launch_gemm_skinny(g, pl.waves, pl.splits, static_cast<float *>(g.workspace), stream);
    case GemmVariant::Generic:
    default:
      return launch_generic<0, OUT>(g, stream);  // replaced below for W4A16
  }
}

// W4A4 plans are instantiated per A block size; W4A16 has no A scales
template <int OUT>
static hipError_t run_plan_blk(const GemmArgs &g, const GemmPlan &pl, hipStream_t stream) {
  if (g.mode == 0 && g.a_blk == 32) return run_plan<OUT, 32>(g, pl, stream);
  if (g.mode == 0 && g.a_blk == 64) return run_plan<OUT, 64>(g, pl, stream);
  return run_plan<OUT, 16>(g, pl, stream);
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream) {
  const GemmPlan pl = plan_gemm(g.mode, g.M, g.N, g.K, g.lda);
  if (g.out_dtype == 2) {
    // NVFP4 output: the tile kernels requantize in their epilogue (or in the split-K reduction);
    // the generic kernel writes scaled fp32 into the workspace and the reduction pass requantizes
    if (pl.variant == GemmVariant::Generic) {
      GemmArgs f = g;
      f.c = g.workspace;
      f.ldc = g.N;
      f.out_dtype = 0;
      hipError_t e = g.mode == 0 ? launch_generic<0, 0>(f, stream) : launch_generic<1, 0>(f, stream);
      if (e != hipSuccess) return e;
      return launch_splitk_reduce(static_cast<const float *>(g.workspace), 1, g.M, g.N, nullptr, 2, 0, nullptr,
                                  nullptr, g.qo, stream);
    }
    return run_plan_blk<2>(g, pl, stream);
  }
  if (pl.variant == GemmVariant::Generic) {
    if (g.mode == 0) return g.out_dtype == 0 ? launch_generic<0, 0>(g, stream) : launch_generic<0, 1>(g, stream);
    return g.out_dtype == 0 ? launch_generic<1, 0>(g, stream) : launch_generic<1, 1>(g, stream);
  }
  return g.out_dtype == 0 ? run_plan_blk<0>(g, pl, stream) : run_plan_blk<1>(g, pl, stream);
}

}  // namespace nvfp4
