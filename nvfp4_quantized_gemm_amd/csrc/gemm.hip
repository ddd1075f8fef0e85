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
// Kernel structure (k_gemm_tiled): a 256-thread workgroup (4 waves) owns a BM x BN tile and walks
// K in chunks of 128.  Per chunk it stages, through registers, A codes + A scale bytes (or bf16 A)
// and one prepacked B unit per 32 columns into an LDS buffer (double-buffered: one barrier per
// chunk).  Each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  For MFMA step s
// (16 k) lane l = r + 32 h takes k in [64 h + 8 s, +8): that is dword s of the lane's 32-byte code
// run, so A and B codes are read with 16-byte LDS loads and the k permutation is the same on both
// sides.  Dequantization in registers: v_cvt_scalef32_pk_{f16,f32}_fp4 with scale 1 gives exact q;
// one multiply by the block's E4M3 scale gives q * e.  The epilogue multiplies the fp32
// accumulator by S_A * S_B and converts.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kChunk = 128;  // k per LDS stage

template <int MODE, int BM, int BN>
struct TileCfg {
  static constexpr int kALds = (MODE == 0) ? BM * 64 : BM * 256;  // codes or bf16
  static constexpr int kASLds = (MODE == 0) ? BM * 8 : 0;
  static constexpr int kBLds = BN * 64;
  static constexpr int kBSLds = BN * 8;
  static constexpr int kStage = kALds + kASLds + kBLds + kBSLds;
  static constexpr int kAIters = (MODE == 0) ? (BM * 4) / 256 : (BM * 16) / 256;  // 16-B loads per thread
  static constexpr int kBIters = (BN * 128) / (32 * 256);                          // BN/32 units x 128 chunks
  static constexpr int kBSChunks = BN / 2;                                          // 16-B chunks of B scales
};

__device__ __forceinline__ f16x8 dequant_f16x8(uint32_t codes, _Float16 e) {
  const f16x2 ee = {e, e};
  const f16x2 q[4] = {fp4_decode2_f16<0>(codes) * ee, fp4_decode2_f16<1>(codes) * ee,
                      fp4_decode2_f16<2>(codes) * ee, fp4_decode2_f16<3>(codes) * ee};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = q[j].x;
    r[2 * j + 1] = q[j].y;
  }
  return r;
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

// MODE 0 = W4A4 (fp16 MFMA), 1 = W4A16 (bf16 MFMA).  WM x WN waves.
template <int MODE, int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_tiled(
    const void *__restrict__ a, const uint8_t *__restrict__ a_scales, const float *__restrict__ a_ts,
    const uint8_t *__restrict__ bp, const float *__restrict__ b_ts, int M, int N, int K, int64_t lda,
    void *__restrict__ c, int64_t ldc, int tiles_m, int tiles_n) {
  using Cfg = TileCfg<MODE, BM, BN>;
  constexpr int TM = BM / WM / 32;  // MFMA tiles per wave along M
  constexpr int TN = BN / WN / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // XCD-aware tile order: consecutive dispatches land on different XCDs; give each XCD a
  // contiguous range of tiles (row-major over the tile grid) so its L2 sees shared A rows.
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int full = (ntiles / 8) * 8;  // bijective remap on the multiple-of-8 prefix
    if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  }
  const int tile_m = bid / tiles_n, tile_n = bid % tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int Kc = K / kChunk;
  const int64_t Nu = ((int64_t)N + 31) / 32;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;

  // ---- global -> register staging -------------------------------------------------------------
  u32x4 ra[Cfg::kAIters];
  uint32_t ras[2];
  u32x4 rb[Cfg::kBIters];
  u32x4 rbs;

  auto load_chunk = [&](int kc) {
    if (MODE == 0) {
      const uint8_t *A = static_cast<const uint8_t *>(a);
#pragma unroll
      for (int it = 0; it < Cfg::kAIters; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 2, cq = idx & 3;
        const int64_t row = m0 + r;
        if (row < M) ra[it] = *reinterpret_cast<const u32x4 *>(A + row * (lda / 2) + kc * 64 + 16 * cq);
        else ra[it] = (u32x4){0u, 0u, 0u, 0u};
      }
      if (tid < BM) {
        const int64_t row = m0 + tid;
        if (row < M) {
          const u32x2 s = *reinterpret_cast<const u32x2 *>(a_scales + row * (lda / 16) + kc * 8);
          ras[0] = s.x;
          ras[1] = s.y;
        } else {
          ras[0] = ras[1] = 0u;
        }
      }
    } else {
      const uint16_t *A = static_cast<const uint16_t *>(a);
#pragma unroll
      for (int it = 0; it < Cfg::kAIters; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 4, cq = idx & 15;
        const int64_t row = m0 + r;
        if (row < M) ra[it] = *reinterpret_cast<const u32x4 *>(A + row * lda + (int64_t)kc * kChunk + 8 * cq);
        else ra[it] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int it = 0; it < Cfg::kBIters; ++it) {
      const int idx = it * 256 + tid;
      const int u = idx >> 7, off = idx & 127;
      const int64_t nu = n0 / 32 + u;
      if (nu < Nu)
        rb[it] = *reinterpret_cast<const u32x4 *>(bp + ((uint64_t)nu * Kc + kc) * 2048ull + 16ull * off);
      else
        rb[it] = (u32x4){0u, 0u, 0u, 0u};
    }
    if (tid < Cfg::kBSChunks) {
      const int u = tid >> 4, off = tid & 15;
      const int64_t nu = n0 / 32 + u;
      if (nu < Nu)
        rbs = *reinterpret_cast<const u32x4 *>(bp + scale_region + ((uint64_t)nu * Kc + kc) * 256ull + 16ull * off);
      else
        rbs = (u32x4){0u, 0u, 0u, 0u};
    }
  };

  auto store_chunk = [&](int buf) {
    uint8_t *st = smem + buf * Cfg::kStage;
    uint8_t *sA = st, *sAS = st + Cfg::kALds, *sB = sAS + Cfg::kASLds, *sBS = sB + Cfg::kBLds;
    if (MODE == 0) {
#pragma unroll
      for (int it = 0; it < Cfg::kAIters; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 2, cq = idx & 3;
        const int sub = r >> 5, ln = (r & 31) + 32 * (cq >> 1), part = cq & 1;
        *reinterpret_cast<u32x4 *>(sA + ((sub * 2 + part) * 64 + ln) * 16) = ra[it];
      }
      if (tid < BM) {
        const int sub = tid >> 5, ln = tid & 31;
        *reinterpret_cast<uint32_t *>(sAS + (sub * 64 + ln) * 4) = ras[0];
        *reinterpret_cast<uint32_t *>(sAS + (sub * 64 + ln + 32) * 4) = ras[1];
      }
    } else {
#pragma unroll
      for (int it = 0; it < Cfg::kAIters; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 4, cq = idx & 15;  // cq: 16-B piece (8 k) of the row's 128 k
        const int sub = r >> 5, h = cq >> 3, s = cq & 7;
        const int ln = (r & 31) + 32 * h;
        *reinterpret_cast<u32x4 *>(sA + ((sub * 8 + s) * 64 + ln) * 16) = ra[it];
      }
    }
#pragma unroll
    for (int it = 0; it < Cfg::kBIters; ++it) {
      const int idx = it * 256 + tid;
      *reinterpret_cast<u32x4 *>(sB + idx * 16) = rb[it];
    }
    if (tid < Cfg::kBSChunks) *reinterpret_cast<u32x4 *>(sBS + tid * 16) = rbs;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_chunk(0);
  store_chunk(0);
  __syncthreads();

  for (int kc = 0; kc < Kc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < Kc) load_chunk(kc + 1);

    const uint8_t *st = smem + buf * Cfg::kStage;
    const uint8_t *sA = st, *sAS = st + Cfg::kALds, *sB = sAS + Cfg::kASLds, *sBS = sB + Cfg::kBLds;

    // per-chunk scale registers
    uint32_t bsw[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int unit = (wn * (BN / WN)) / 32 + j;
      bsw[j] = *reinterpret_cast<const uint32_t *>(sBS + (unit * 64 + lane) * 4);
    }
    uint32_t asw[TM];
    if (MODE == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int sub = (wm * (BM / WM)) / 32 + i;
        asw[i] = *reinterpret_cast<const uint32_t *>(sAS + (sub * 64 + lane) * 4);
      }
    }

#pragma unroll
    for (int p = 0; p < 2; ++p) {  // two parts of 4 MFMA steps each
      u32x4 bc[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int unit = (wn * (BN / WN)) / 32 + j;
        bc[j] = *reinterpret_cast<const u32x4 *>(sB + ((unit * 2 + p) * 64 + lane) * 16);
      }
      u32x4 ac[TM];
      if (MODE == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int sub = (wm * (BM / WM)) / 32 + i;
          ac[i] = *reinterpret_cast<const u32x4 *>(sA + ((sub * 2 + p) * 64 + lane) * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = 4 * p + q;    // MFMA step within the chunk
        const int blk = s >> 1;     // lane's scale block (of its 4) for this step
        if (MODE == 0) {
          f16x8 af[TM], bf[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const _Float16 e = (_Float16)e4m3_to_f32((asw[i] >> (8 * blk)) & 0xffu);
            af[i] = dequant_f16x8(ac[i][q], e);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const _Float16 e = (_Float16)e4m3_to_f32((bsw[j] >> (8 * blk)) & 0xffu);
            bf[j] = dequant_f16x8(bc[j][q], e);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        } else {
          bf16x8 af[TM], bf[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int sub = (wm * (BM / WM)) / 32 + i;
            const u32x4 w = *reinterpret_cast<const u32x4 *>(sA + ((sub * 8 + s) * 64 + lane) * 16);
            af[i] = __builtin_bit_cast(bf16x8, w);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const float e = e4m3_to_f32((bsw[j] >> (8 * blk)) & 0xffu);
            bf[j] = dequant_bf16x8(bc[j][q], e);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }

    if (kc + 1 < Kc) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: scale by S_A * S_B, convert, store ---------------------------------------------
  const float sab = (MODE == 0) ? (*a_ts) * (*b_ts) : *b_ts;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * (BM / WM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M) store_out<OUT>(c, ldc, row, col, acc[i][j][v] * sab);
      }
    }
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
                                                      int64_t lda, void *__restrict__ c, int64_t ldc) {
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
        av = q.x * e4m3_to_f32(a_scales[m * (lda / 16) + (k >> 4)]);
      } else {
        av = __uint_as_float((uint32_t) static_cast<const uint16_t *>(a)[m * lda + k] << 16);
      }
      acc = fmaf(av, prepacked_weight(bp, Kc, scale_region, n, k), acc);
    }
    store_out<OUT>(c, ldc, m, n, acc * sab);
  }
}

// ---- launchers ----------------------------------------------------------------------------------

template <int MODE, int BM, int BN, int WM, int WN, int OUT>
static hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
  using Cfg = TileCfg<MODE, BM, BN>;
  const int tm = (int)((g.M + BM - 1) / BM), tn = (int)((g.N + BN - 1) / BN);
  auto kern = k_gemm_tiled<MODE, BM, BN, WM, WN, OUT>;
  const int smem = 2 * Cfg::kStage;
  static bool configured = false;  // per instantiation
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    configured = true;
  }
  kern<<<tm * tn, 256, smem, stream>>>(g.a, g.a_scales, g.a_ts, static_cast<const uint8_t *>(g.b), g.b_ts,
                                       (int)g.M, (int)g.N, (int)g.K, g.lda, g.c, g.ldc, tm, tn);
  return hipGetLastError();
}

template <int MODE, int OUT>
static hipError_t launch_generic(const GemmArgs &g, hipStream_t stream) {
  int64_t total = g.M * g.N;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  k_gemm_generic<MODE, OUT><<<(unsigned)grid, 256, 0, stream>>>(g.a, g.a_scales, g.a_ts,
                                                                 static_cast<const uint8_t *>(g.b), g.b_ts, g.M, g.N,
                                                                 g.K, g.lda, g.c, g.ldc);
  return hipGetLastError();
}

GemmVariant select_gemm_variant(int mode, int64_t M, int64_t N, int64_t K, int64_t lda) {
  if (K % kChunk != 0) return GemmVariant::Generic;
  if (mode == 0) {
    if (lda % kChunk != 0) return GemmVariant::Generic;
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    return (t256 >= 240) ? GemmVariant::W4A4_256x256 : GemmVariant::W4A4_128x128;
  }
  return GemmVariant::W4A16_128x256;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream) {
  const GemmVariant v = select_gemm_variant(g.mode, g.M, g.N, g.K, g.lda);
  const bool f32 = (g.out_dtype == 0);
  switch (v) {
    case GemmVariant::W4A4_256x256:
      return f32 ? launch_tiled<0, 256, 256, 2, 2, 0>(g, stream) : launch_tiled<0, 256, 256, 2, 2, 1>(g, stream);
    case GemmVariant::W4A4_128x128:
      return f32 ? launch_tiled<0, 128, 128, 2, 2, 0>(g, stream) : launch_tiled<0, 128, 128, 2, 2, 1>(g, stream);
    case GemmVariant::W4A16_128x256:
      return f32 ? launch_tiled<1, 128, 256, 1, 4, 0>(g, stream) : launch_tiled<1, 128, 256, 1, 4, 1>(g, stream);
    case GemmVariant::Generic:
    default:
      if (g.mode == 0) return f32 ? launch_generic<0, 0>(g, stream) : launch_generic<0, 1>(g, stream);
      return f32 ? launch_generic<1, 0>(g, stream) : launch_generic<1, 1>(g, stream);
  }
}

}  // namespace nvfp4

namespace nvfp4 {
size_t gemm_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }
}  // namespace nvfp4
