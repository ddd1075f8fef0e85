// Weight-only NVFP4 GEMM for few activation rows (W4A16, M <= 32): Y = A B^T with A bf16 [M][K]
// and B an NVFP4 weight in the prepacked layout [NVFP4-DiT page, Methodology section 3; vllm-omni
// NVFP4 RFC, Open Question 1: weight-only NVFP4].  With M this small the call streams the packed
// weight once (0.5625 B per weight element) and is bound by HBM bandwidth, not by matrix math.
//
// Work split: workgroup (unit u, split s) owns the 32 output columns of prepacked unit u and the
// 128-k chunks [s Kc / S, (s + 1) Kc / S); its NW waves (4, 8 or 16) take every NW-th chunk of
// that range.  Per chunk a lane loads its two 16-byte code parts and
// 4 scale bytes of the unit (the prepacked order is the MFMA operand order) plus its A row segment
// and runs 8 bf16 MFMA steps with the weight fragment as the row operand: lane l = r + 32 h then
// ends with output row m = r and, per group g, columns 8 g + 4 h + 0..3.  Rows r >= M load nothing
// and contribute zeros.  Weight loads run three chunks ahead; each activation step slot is
// reloaded for the next chunk as soon as its MFMA has consumed it.
// The waves' accumulators are added in LDS in wave order (deterministic).  With S = 1 (wide N)
// one kernel produces the output; narrow N splits K over S workgroups per unit so that enough
// workgroups stream, and the split-K reduction kernel adds the S fp32 partials in order.
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

}  // namespace

template <int OUT, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_skinny(const uint16_t *__restrict__ a, int64_t lda,
                                                         const uint8_t *__restrict__ bp,
                                                         const float *__restrict__ b_ts, int M, int N, int K,
                                                         void *__restrict__ c, int64_t ldc, int splits,
                                                         float *__restrict__ partial) {
  __shared__ float red[NW][16][64];
  const int Kc = K / 128, Nu = (N + 31) / 32;
  const int u = blockIdx.x % Nu, split = blockIdx.x / Nu;
  const int kb = (int)((int64_t)split * Kc / splits), ke = (int)((int64_t)(split + 1) * Kc / splits);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  const uint8_t *bcode = bp + (uint64_t)u * (uint64_t)Kc * 2048ull + lane * 16;
  const uint8_t *bscale = bp + scale_region + (uint64_t)u * (uint64_t)Kc * 256ull + lane * 4;
  const bool has_row = r < M;
  const uint16_t *arow = a + (int64_t)(has_row ? r : 0) * lda + 64 * h;

  struct BRegs {
    u32x4 code[2];  // parts 0 and 1: dword s & 3 of part s >> 2 holds MFMA step s
    uint32_t sc;    // the lane's four E4M3 block scales
  };
  auto load_b = [&](int kc, BRegs &x) {
    const uint8_t *pc = bcode + (uint64_t)kc * 2048ull;
    x.code[0] = load16<true>(pc);  // streaming: each weight byte is read once per call
    x.code[1] = load16<true>(pc + 1024);
    x.sc = *reinterpret_cast<const uint32_t *>(bscale + (uint64_t)kc * 256ull);
  };
  auto load_a = [&](int kc, u32x4 *x) {
    const uint16_t *pa = arow + (int64_t)kc * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      x[s] = has_row ? *reinterpret_cast<const u32x4 *>(pa + 8 * s) : z;
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc0[v] = 0.0f;
    acc1[v] = 0.0f;
  }
  // wave w takes chunks w, w + NW, ...; weight loads run two chunks ahead, activation loads one
  // wave w takes chunks w, w + NW, ...  Weight loads go into a 3-slot ring (slot j holds chunks
  // i = j mod 3 of the wave's sequence; a slot is refilled three chunks ahead right after use; the
  // loop is unrolled by 3 so slots never move between registers, which would wait on the loads).
  if (kb + wave < ke) {
    BRegs b[3];
    u32x4 av[8];
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (kb + wave + j * NW < ke) load_b(kb + wave + j * NW, b[j]);
    load_a(kb + wave, av);
#pragma unroll 1
    for (int i0 = 0; kb + wave + i0 * NW < ke; i0 += 3) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int kc = kb + wave + (i0 + j) * NW;
        if (kc < ke) {
          const bool more = kc + NW < ke;
          float e[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) e[t] = e4m3_to_f32((b[j].sc >> (8 * t)) & 0xffu);
          const uint16_t *pa_next = arow + (int64_t)(kc + NW) * 128;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const bf16x8 bf = dequant_b(b[j].code[s >> 2][s & 3], e[s >> 1]);
            const bf16x8 af = __builtin_bit_cast(bf16x8, av[s]);
            if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc1, 0, 0, 0);
            else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc0, 0, 0, 0);
            // rolling activation prefetch: this step's slot now loads the next chunk's step
            if (more && has_row) av[s] = *reinterpret_cast<const u32x4 *>(pa_next + 8 * s);
          }
          if (kc + 3 * NW < ke) load_b(kc + 3 * NW, b[j]);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc0[v] + acc1[v];
  __syncthreads();
  if (wave >= 4) return;

  // wave w < 4 finishes column group g = w: columns n = 32 u + 8 w + 4 h + j, row m = r; the
  // waves' partial sums are added in wave order (deterministic)
  float out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = 4 * wave + j;
    float sum = red[0][v][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][v][lane];
    out[j] = sum;
  }
  if (!has_row) return;
  const int n = 32 * u + 8 * wave + 4 * h;
  if (OUT == 2 || splits > 1) {
    // unscaled fp32 partial; the split-K reduction sums the splits in order, scales and converts
    // (OUT 2, NVFP4 output: always, the reduction pass requantizes)
    float *dst = partial + (int64_t)split * M * N + (int64_t)r * N + n;
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
    float *dst = static_cast<float *>(c) + (int64_t)r * ldc + n;
    if (n + 3 < N && (ldc % 4) == 0) {
      const f32x4 o = {out[0] * sb, out[1] * sb, out[2] * sb, out[3] * sb};
      *reinterpret_cast<f32x4 *>(dst) = o;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) dst[j] = out[j] * sb;
    }
  } else {
    __bf16 *dst = static_cast<__bf16 *>(c) + (int64_t)r * ldc + n;
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
}

template <int OUT>
static hipError_t launch_skinny_out(const GemmArgs &g, int nw, int splits, float *partial, hipStream_t stream) {
  const int Nu = (int)((g.N + 31) / 32);
  const unsigned grid = (unsigned)(Nu * splits);
  const uint16_t *a = static_cast<const uint16_t *>(g.a);
  const uint8_t *b = static_cast<const uint8_t *>(g.b);
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
  if (nw >= 16)
    k_gemm_skinny<OUT, 16><<<grid, 1024, 0, stream>>>(a, g.lda, b, g.b_ts, M, N, K, g.c, g.ldc, splits, partial);
  else if (nw >= 8)
    k_gemm_skinny<OUT, 8><<<grid, 512, 0, stream>>>(a, g.lda, b, g.b_ts, M, N, K, g.c, g.ldc, splits, partial);
  else
    k_gemm_skinny<OUT, 4><<<grid, 256, 0, stream>>>(a, g.lda, b, g.b_ts, M, N, K, g.c, g.ldc, splits, partial);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmArgs &g, int waves, int splits, float *partial, hipStream_t stream) {
  hipError_t e = g.out_dtype == 0   ? launch_skinny_out<0>(g, waves, splits, partial, stream)
                 : g.out_dtype == 1 ? launch_skinny_out<1>(g, waves, splits, partial, stream)
                                    : launch_skinny_out<2>(g, waves, splits, partial, stream);
  if (e != hipSuccess || (splits == 1 && g.out_dtype != 2)) return e;
  return launch_splitk_reduce(partial, splits, g.M, g.N, g.c, g.out_dtype, g.ldc, nullptr, g.b_ts, g.qo, stream);
}

}  // namespace nvfp4
