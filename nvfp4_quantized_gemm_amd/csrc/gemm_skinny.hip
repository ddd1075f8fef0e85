// Weight-only NVFP4 GEMM for few activation rows (W4A16, M <= 32): Y = A B^T with A bf16 [M][K]
// and B an NVFP4 weight in the prepacked layout [NVFP4-DiT page, Methodology section 3; vllm-omni
// NVFP4 RFC, Open Question 1: weight-only NVFP4].  With M this small the call streams the packed
// weight once (0.5625 B per weight element) and is bound by HBM bandwidth, not by matrix math.
//
// Work split: workgroup (unit u, split s) owns the 32 output columns of prepacked unit u and the
// K chunks [s Kc / S, (s + 1) Kc / S); its four waves take every fourth chunk of that range.  Per
// chunk a lane loads its two 16-byte code parts and 4 scale bytes of the unit (the prepacked order
// is the MFMA operand order) plus its A row segment, and runs 8 bf16 MFMA steps with the weight
// fragment as the row operand: lane l = r + 32 h then ends with output row m = r and, per group g,
// columns 8 g + 4 h + 0..3.  Rows r >= M load nothing and contribute zeros.  The next chunk's loads
// are issued before the current chunk's math.  The four waves' accumulators are summed in LDS in a
// fixed order; with S > 1 the workgroup writes an fp32 partial and the split-K reduction kernel
// sums the S partials in order (deterministic), scales by S_B and converts.
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

struct ChunkRegs {
  u32x4 code[2];  // parts 0 and 1: dword s & 3 of part s >> 2 holds MFMA step s
  uint32_t sc;    // the lane's four E4M3 block scales
  u32x4 a[8];     // A row segment: 8 bf16 per step
};

}  // namespace

template <int OUT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t *__restrict__ a, int64_t lda,
                                                     const uint8_t *__restrict__ bp, const float *__restrict__ b_ts,
                                                     int M, int N, int K, void *__restrict__ c, int64_t ldc, int splits,
                                                     float *__restrict__ partial) {
  __shared__ float red[4][16][64];
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

  auto load = [&](int kc, ChunkRegs &x) {
    const uint8_t *pc = bcode + (uint64_t)kc * 2048ull;
    x.code[0] = *reinterpret_cast<const u32x4 *>(pc);
    x.code[1] = *reinterpret_cast<const u32x4 *>(pc + 1024);
    x.sc = *reinterpret_cast<const uint32_t *>(bscale + (uint64_t)kc * 256ull);
    const uint16_t *pa = arow + (int64_t)kc * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      x.a[s] = has_row ? *reinterpret_cast<const u32x4 *>(pa + 8 * s) : z;
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc0[v] = 0.0f;
    acc1[v] = 0.0f;
  }
  int kc = kb + wave;
  if (kc < ke) {
    ChunkRegs cur, nxt;
    load(kc, cur);
    for (; kc < ke; kc += 4) {
      if (kc + 4 < ke) load(kc + 4, nxt);
      float e[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) e[t] = e4m3_to_f32((cur.sc >> (8 * t)) & 0xffu);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 bf = dequant_b(cur.code[s >> 2][s & 3], e[s >> 1]);
        const bf16x8 af = __builtin_bit_cast(bf16x8, cur.a[s]);
        if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc0, 0, 0, 0);
      }
      if (kc + 4 < ke) cur = nxt;
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc0[v] + acc1[v];
  __syncthreads();

  // wave w finishes column group g = w: columns n = 32 u + 8 w + 4 h + j, row m = r
  float out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = 4 * wave + j;
    out[j] = ((red[0][v][lane] + red[1][v][lane]) + red[2][v][lane]) + red[3][v][lane];
  }
  if (!has_row) return;
  const int n = 32 * u + 8 * wave + 4 * h;
  if (splits > 1) {
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

hipError_t launch_gemm_skinny(const GemmArgs &g, int splits, float *partial, hipStream_t stream) {
  const int Nu = (int)((g.N + 31) / 32);
  const int64_t grid = (int64_t)Nu * splits;
  const uint16_t *a = static_cast<const uint16_t *>(g.a);
  const uint8_t *b = static_cast<const uint8_t *>(g.b);
  if (g.out_dtype == 0)
    k_gemm_skinny<0><<<(unsigned)grid, 256, 0, stream>>>(a, g.lda, b, g.b_ts, (int)g.M, (int)g.N, (int)g.K, g.c,
                                                        g.ldc, splits, partial);
  else
    k_gemm_skinny<1><<<(unsigned)grid, 256, 0, stream>>>(a, g.lda, b, g.b_ts, (int)g.M, (int)g.N, (int)g.K, g.c,
                                                        g.ldc, splits, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(partial, splits, g.M, g.N, g.c, g.out_dtype, g.ldc, nullptr, g.b_ts, stream);
}

}  // namespace nvfp4
