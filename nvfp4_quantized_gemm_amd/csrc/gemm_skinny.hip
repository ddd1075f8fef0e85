// Weight-only NVFP4 GEMM for few activation rows (W4A16, M <= 64): Y = A B^T with A bf16 [M][K]
// and B an NVFP4 weight in the prepacked layout [NVFP4-DiT page, Methodology section 3; vllm-omni
// NVFP4 RFC, Open Question 1: weight-only NVFP4].  With M this small the call streams the packed
// weight once (0.5625 B per weight element) and is bound by HBM bandwidth, not by matrix math.
//
// Work split: workgroup (unit u, split s) owns the 32 output columns of prepacked unit u and the
// 128-k chunks [s Kc / S, (s + 1) Kc / S); its NW waves (4, 8 or 16) take every NW-th chunk of
// that range.  Per chunk a lane loads its two 16-byte code parts and 4 scale bytes of the unit (the
// prepacked order is the MFMA operand order) and runs 8 bf16 MFMA steps with the weight fragment
// as the row operand and activation row r in lane l = r + 32 h: the lane ends with output row
// m = r and, per group g, columns 8 g + 4 h + 0..3.  Rows r >= M are computed from duplicate rows
// and never stored.  Weight loads run three chunks ahead in registers.
//
// Activations: in the MFMA operand order every lane holds a different row, so loading them in that
// order touches 64 cache lines per instruction.  Instead each wave copies its chunk of the first
// MR rows (MR = M rounded up to 4, 8, 16, 32 or 64; 256 bytes per row) straight into a
// wave-private LDS ring with row-contiguous 16-byte DMAs (16 lanes per row), L chunks ahead (L = 3,
// 3, 2, 1, 1 by MR, which keeps two workgroups of 8 waves, or of 4 waves for 64 rows, per CU), and
// reads the operand order back from there; 64 rows are two MFMA column operands of 32 rows.
// The 16-byte pieces of row r are stored XOR-swizzled by r % 16, so that the 16 lanes of each read
// pass hit 16 different bank groups.
// The waves' accumulators are added in LDS in wave order (deterministic).  With S = 1 (wide N)
// one kernel produces the output; narrow N splits K over S workgroups per unit so that enough
// workgroups stream, and the split-K reduction kernel adds the S fp32 partials in order.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

__device__ __forceinline__ bf16x8 dequant_b(uint32_t codes, float e) {
  const f32x2 q0 = fp4_decode2_f32<0>(codes), q1 = fp4_decode2_f32<1>(codes);
  const f32x2 q2 = fp4_decode2_f32<2>(codes), q3 = fp4_decode2_f32<3>(codes);
  bf16x8 r;
  r[0] = (__bf16)(q0.x * e);
  r[1] = (__bf16)(q0.y * e);
  r[2] = (__bf16)(q1.x * e);
  r[3] = (__bf16)(q1.y * e);
  r[4] = (__bf16)(q2.x * e);
  r[5] = (__bf16)(q2.y * e);
  r[6] = (__bf16)(q3.x * e);
  r[7] = (__bf16)(q3.y * e);
  return r;
}

// Activation ring of one wave: L slots of one chunk of MR rows each; MR / 4 DMAs fill a slot.
// MR = 64 holds two groups of 32 rows, each its own MFMA column operand.
template <int MR>
struct SkinnyA {
  static_assert(MR == 4 || MR == 8 || MR == 16 || MR == 32 || MR == 64, "row classes");
  static constexpr int kL = (MR <= 8) ? 3 : (MR == 16 ? 2 : 1);
  static constexpr int kSlot = MR * 256;
  static constexpr int kDma = MR / 4;
  static constexpr int kGroups = MR > 32 ? MR / 32 : 1;
};

template <int NW, int MR>
constexpr int skinny_lds_bytes() {
  constexpr int ring = NW * SkinnyA<MR>::kL * SkinnyA<MR>::kSlot;
  constexpr int red = NW * SkinnyA<MR>::kGroups * 16 * 64 * 4;
  return ring > red ? ring : red;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// keeps the vector-memory issue order as written (the waits above count operations in that order)
__device__ __forceinline__ void issue_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

// waves per SIMD: 1.5 workgroups per CU of 8 or 16 waves need 4; the 64-row class runs 4-wave
// workgroups two per CU and needs the registers of a second row group
template <int OUT, int NW, int MR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MR > 32 ? 2 : 4))) void k_gemm_skinny(const uint16_t *__restrict__ a, int64_t lda,
                                                         const uint8_t *__restrict__ bp,
                                                         const float *__restrict__ b_ts, int M, int N, int K,
                                                         void *__restrict__ c, int64_t ldc, int splits,
                                                         float *__restrict__ partial) {
  using SA = SkinnyA<MR>;
  constexpr int L = SA::kL, RG = SA::kGroups;
  constexpr int NB = 3;            // vector-memory operations of one chunk's weight loads
  constexpr int NA = SA::kDma;     // ... and of one chunk's activation DMAs
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int Kc = K / 128, Nu = (N + 31) / 32;
  const int u = blockIdx.x % Nu, split = blockIdx.x / Nu;
  const int kb = (int)((int64_t)split * Kc / splits), ke = (int)((int64_t)(split + 1) * Kc / splits);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  // wave-uniform bases + 32-bit lane offsets (the loads take the scalar-base form)
  const uint8_t *bcode = bp + (uint64_t)u * (uint64_t)Kc * 2048ull;
  const uint8_t *bscale = bp + scale_region + (uint64_t)u * (uint64_t)Kc * 256ull;
  const uint32_t lcode = (uint32_t)lane * 16u, lscale = (uint32_t)lane * 4u;

  // DMA q of a chunk: lane l takes row 4 q + l / 16 (rows past M re-read row M - 1) and lands at
  // LDS unit 64 q + l of the slot, i.e. row-major 256-byte rows holding piece (l % 16) ^ (row % 16).
  // Lane-dependent offsets are recomputed per chunk from an opaque copy of the lane index (a few
  // VALU operations) rather than kept live across the loop.
  // (byte offsets within a chunk column: 32 lda < 2^31 is a condition of this kernel's plan)
  uint8_t *aring = smem + wave * (L * SA::kSlot);

  struct BRegs {
    u32x4 code[2];  // parts 0 and 1: dword s & 3 of part s >> 2 holds MFMA step s
    uint32_t sc;    // the lane's four E4M3 block scales
  };
  auto load_b = [&](int kc, BRegs &x) {
    const uint8_t *pc = bcode + (uint64_t)kc * 2048ull;
    x.code[0] = load16<true>(pc + lcode);  // streaming: each weight byte is read once per call
    x.code[1] = load16<true>(pc + (lcode + 1024u));
    x.sc = *reinterpret_cast<const uint32_t *>(bscale + (uint64_t)kc * 256ull + lscale);
  };
  // wave w takes chunks kb + w + i NW, i = 0 .. nw - 1
  const int nw = (kb + wave < ke) ? (ke - kb - wave + NW - 1) / NW : 0;
  auto chunk_of = [&](int i) { return kb + wave + i * NW; };

  // one row group: two accumulators alternate between the steps; two row groups: one each, the
  // groups alternating within a step (either way no MFMA waits on the one before it)
  f32x16 acc[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc[0][v] = 0.0f;
    acc[1][v] = 0.0f;
  }
  // Issue order, chunk i: activation DMAs of chunk i + L into the slot chunk i has just read, then
  // weight loads of chunk i + 3 into register slot i % 3 (the loop is unrolled by 3 so slots never
  // move between registers); the prologue issues the same pattern for the virtual chunks -3 .. -1,
  // and nothing past the wave's last chunk is issued.  So when chunk i starts, the operations
  // issued after its activation DMAs are the weight loads of the chunks i - L + 3 .. i + 2 and the
  // DMAs of the chunks i + 1 .. i + L - 1 that exist: with t = nw - i chunks left, L weight groups
  // and L - 1 DMA groups for t >= 3, L - 1 and min(1, L - 1) for t = 2, max(L - 2, 0) and none
  // for t = 1.
  if (nw > 0) {
    BRegs b[3];
    auto issue_a = [&](int i, int slot) {  // the wave's chunk i into ring slot `slot`
      const uint8_t *src = reinterpret_cast<const uint8_t *>(a) + (int64_t)chunk_of(i) * 256;
      uint8_t *dst = aring + slot * SA::kSlot;
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int q = 0; q < SA::kDma; ++q) {
        const int row = 4 * q + (ln >> 4);
        const uint32_t off = 2u * ((uint32_t)min(row, M - 1) * (uint32_t)lda) + 16u * (uint32_t)((ln & 15) ^ (row & 15));
        g2l16(src + off, dst + q * 1024);
      }
    };
#pragma unroll
    for (int v = -3; v < 0; ++v) {
      if (v + L >= 0 && v + L < nw) issue_a(v + L, v + L);
      issue_order();
      if (v + 3 < nw) load_b(chunk_of(v + 3), b[v + 3]);
      issue_order();
    }
    // chunk i with its weights in register slot J
    auto body = [&](int i, auto slot_tag) {
      constexpr int J = decltype(slot_tag)::value;
      {
        const int t = nw - i;
        constexpr int L2 = (L >= 2) ? L - 2 : 0, NA2 = (L >= 2) ? NA : 0;
        if (t >= 3) wait_vmcnt<L * NB + (L - 1) * NA>();
        else if (t == 2) wait_vmcnt<(L - 1) * NB + NA2>();
        else wait_vmcnt<L2 * NB>();
      }
      const int sl = i % L;
      // operand read of step s: row r % MR, piece 8 h + s, i.e. 16-byte unit (8 h + s) ^ (r % 16)
      // of the row = ((8 h) ^ (r % 16)) ^ s
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int rrow = ln & 31 & (MR - 1), y = (8 * (ln >> 5)) ^ (rrow & 15);
      const uint8_t *rd = aring + sl * SA::kSlot + rrow * 256;
      u32x4 av[RG][8];  // group g: rows 32 g + r, 32 rows = 8 KB further in the slot
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int s = 0; s < 8; ++s) av[g][s] = *reinterpret_cast<const u32x4 *>(rd + g * 8192 + ((y ^ s) << 4));
      // the slot is refilled next: its reads must have completed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (i + L < nw) issue_a(i + L, sl);
      issue_order();
      float e[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) e[t] = e4m3_to_f32((b[J].sc >> (8 * t)) & 0xffu);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 bf = dequant_b(b[J].code[s >> 2][s & 3], e[s >> 1]);
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          const int k = (RG == 1) ? (s & 1) : g;
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, __builtin_bit_cast(bf16x8, av[g][s]), acc[k], 0, 0, 0);
        }
      }
      issue_order();
      if (i + 3 < nw) load_b(chunk_of(i + 3), b[J]);
      issue_order();
    };
    int i0 = 0;
#pragma unroll 1
    for (; i0 + 3 <= nw; i0 += 3) {
      body(i0, std::integral_constant<int, 0>{});
      body(i0 + 1, std::integral_constant<int, 1>{});
      body(i0 + 2, std::integral_constant<int, 2>{});
    }
    if (i0 < nw) body(i0, std::integral_constant<int, 0>{});
    if (i0 + 1 < nw) body(i0 + 1, std::integral_constant<int, 1>{});
    wait_vmcnt<0>();  // every DMA has landed before the LDS is reused
  }
  // wave w < 4 finishes column group w of row group g: columns n = 32 u + 8 w + 4 h + j, row
  // m = 32 g + r; the waves' partial sums are added in wave order (deterministic)
  auto store_rows = [&](float (*red)[RG][16][64], int g) {
    float out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = 4 * wave + j;
      float sum = red[0][g][v][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][g][v][lane];
      out[j] = sum;
    }
    const int m = 32 * g + r;
    if (m >= M) return;
    const int n = 32 * u + 8 * wave + 4 * h;
    if (OUT == 2 || splits > 1) {
      // unscaled fp32 partial; the split-K reduction sums the splits in order, scales and converts
      // (OUT 2, NVFP4 output: always, the reduction pass requantizes)
      float *dst = partial + (int64_t)split * M * N + (int64_t)m * N + n;
      if (n + 3 < N && (N % 4) == 0) {
        const f32x4 o = {out[0], out[1], out[2], out[3]};
        *reinterpret_cast<f32x4 *>(dst) = o;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) dst[j] = out[j];
      }
      return;
    }
    const float sb = *b_ts;
    if (OUT == 0) {
      float *dst = static_cast<float *>(c) + (int64_t)m * ldc + n;
      if (n + 3 < N && (ldc % 4) == 0) {
        const f32x4 o = {out[0] * sb, out[1] * sb, out[2] * sb, out[3] * sb};
        *reinterpret_cast<f32x4 *>(dst) = o;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) dst[j] = out[j] * sb;
      }
    } else {
      __bf16 *dst = static_cast<__bf16 *>(c) + (int64_t)m * ldc + n;
      if (n + 3 < N && (ldc % 4) == 0) {
        const bf16x2 h0 = {(__bf16)(out[0] * sb), (__bf16)(out[1] * sb)};
        const bf16x2 h1 = {(__bf16)(out[2] * sb), (__bf16)(out[3] * sb)};
        const u32x2 o = {__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
        *reinterpret_cast<u32x2 *>(dst) = o;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) dst[j] = (__bf16)(out[j] * sb);
      }
    }
  };
  // the reduction below reuses the LDS of the activation rings
  __syncthreads();
  float(*red)[RG][16][64] = reinterpret_cast<float(*)[RG][16][64]>(smem);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    if (RG == 1) red[wave][0][v][lane] = acc[0][v] + acc[1][v];
    else
#pragma unroll
      for (int g = 0; g < RG; ++g) red[wave][g][v][lane] = acc[g][v];
  }
  __syncthreads();
  if (wave >= 4) return;
#pragma unroll
  for (int g = 0; g < RG; ++g) store_rows(red, g);
}

template <int OUT, int NW, int MR>
static hipError_t launch_skinny_cfg(const GemmArgs &g, int splits, float *partial, hipStream_t stream) {
  constexpr int smem = skinny_lds_bytes<NW, MR>();
  static std::atomic<bool> configured[kMaxDevices];  // per instantiation and device
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(k_gemm_skinny<OUT, NW, MR>), smem, configured);
  if (e != hipSuccess) return e;
  const int Nu = (int)((g.N + 31) / 32);
  k_gemm_skinny<OUT, NW, MR><<<(unsigned)(Nu * splits), NW * 64, smem, stream>>>(
      static_cast<const uint16_t *>(g.a), g.lda, static_cast<const uint8_t *>(g.b), g.b_ts, (int)g.M, (int)g.N,
      (int)g.K, g.c, g.ldc, splits, partial);
  return hipGetLastError();
}

template <int OUT, int NW>
static hipError_t launch_skinny_rows(const GemmArgs &g, int splits, float *partial, hipStream_t stream) {
  if (g.M <= 4) return launch_skinny_cfg<OUT, NW, 4>(g, splits, partial, stream);
  if (g.M <= 8) return launch_skinny_cfg<OUT, NW, 8>(g, splits, partial, stream);
  if (g.M <= 16) return launch_skinny_cfg<OUT, NW, 16>(g, splits, partial, stream);
  return launch_skinny_cfg<OUT, NW, 32>(g, splits, partial, stream);
}

template <int OUT>
static hipError_t launch_skinny_out(const GemmArgs &g, int nw, int splits, float *partial, hipStream_t stream) {
  // 33..64 rows: two row groups, 4-wave workgroups (the 16 KB activation slot of 8 waves would
  // leave one workgroup per CU)
  if (g.M > 32) return launch_skinny_cfg<OUT, 4, 64>(g, splits, partial, stream);
  if (nw >= 16) return launch_skinny_rows<OUT, 16>(g, splits, partial, stream);
  if (nw >= 8) return launch_skinny_rows<OUT, 8>(g, splits, partial, stream);
  return launch_skinny_rows<OUT, 4>(g, splits, partial, stream);
}

hipError_t launch_gemm_skinny(const GemmArgs &g, int waves, int splits, float *partial, hipStream_t stream) {
  hipError_t e = g.out_dtype == 0   ? launch_skinny_out<0>(g, waves, splits, partial, stream)
                 : g.out_dtype == 1 ? launch_skinny_out<1>(g, waves, splits, partial, stream)
                                    : launch_skinny_out<2>(g, waves, splits, partial, stream);
  if (e != hipSuccess || (splits == 1 && g.out_dtype != 2)) return e;
  return launch_splitk_reduce(partial, splits, g.M, g.N, g.c, g.out_dtype, g.ldc, nullptr, g.b_ts, g.qo, stream);
}

}  // namespace nvfp4
