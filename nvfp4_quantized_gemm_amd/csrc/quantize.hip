// NVFP4 quantization kernels for gfx950.
//
// Definition [NVFP4-DiT page, Methodology section 1, Definition III.1; vllm-omni NVFP4 RFC,
// Motivation]: per 16-value block an E4M3 scale e = nearest E4M3 to amax / (6 S) (ties to even,
// saturating at 448), per value the E2M1 code nearest to v / (e S) (ties to the even code,
// saturating at +-6), sign bit copied from v, two codes per byte, low nibble first.  Decisions are
// taken on the exact real quotients.
//
// Data flow: one thread owns one 16-value block (32 B of bf16 or 64 B of fp32 in, 8 B of codes
// and 1 scale byte out), so a wave streams 2-4 KB of contiguous input and writes 512 B + 64 B.
// Dynamic mode runs k_amax first (per-workgroup partial maxima, no atomics, deterministic); every
// quantize workgroup reduces those partials itself and derives S = RN32(amax / 2688).
//
// Exactness (all fast paths bracket the exact real quotient and fall back when unsure):
//  * Block scale.  With c = 1/(6 S) (fp64, once per workgroup), rl = RN32(amax RN32(c (1 - 2^-20)))
//    and rh = RN32(amax RN32(c (1 + 2^-20))) satisfy rl < amax / (6 S) < rh (a few 2^-24 roundings
//    cannot undo a 2^-20 margin).  The hardware fp32 -> E4M3 conversion rounds to nearest-even and
//    is monotone; after clamping to 448 (saturation) the bytes of rl and rh are equal unless the
//    exact ratio lies within ~2^-19 of a midpoint, and then that common byte is the exact one.
//    Otherwise scale_byte_exact() decides with one fp64 division: the exact quotient differs from
//    any E4M3 midpoint (<= 5 significant bits) by >= 2^-31 relative unless equal to it (amax has 24
//    and 6 S 26 significant bits), so the fp64 rounding (2^-53) neither crosses nor creates one.
//  * Element codes.  inv = rcp(e) * RN32(1/S) is within 3 ulp of 1/(e S); lo = RN32(inv (1 - 2^-20))
//    and hi = RN32(inv (1 + 2^-20)) make the fp32 products v*lo and v*hi bracket v/(e S) strictly.
//    The hardware E2M1 conversion (round-half-even, saturating, sign-preserving) is monotone, so
//    when the two bracketing codes agree that code is the exact one.  A block in which any pair
//    disagrees (a value within ~2^-19 of a decision boundary, e.g. an exact tie) takes the exact
//    path: seven per-block fp32 thresholds U_k from the exact fp64 boundaries t_k e S by directed
//    rounding, code = #{k : |v| >= U_k}.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

// ---- input loading ------------------------------------------------------------------------------

template <int DT>
struct BlockIn;

template <>
struct BlockIn<0> {  // fp32
  __device__ static void load(const void *base, uint64_t elem_off, float v[16]) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + elem_off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 w = p[q];
      v[4 * q + 0] = __uint_as_float(w.x);
      v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z);
      v[4 * q + 3] = __uint_as_float(w.w);
    }
  }
};

template <>
struct BlockIn<1> {  // bf16
  __device__ static void load(const void *base, uint64_t elem_off, float v[16]) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem_off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 w = p[q];
      uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[8 * q + 2 * t] = bf16lo(a[t]);
        v[8 * q + 2 * t + 1] = bf16hi(a[t]);
      }
    }
  }
};

// ---- exact pieces ---------------------------------------------------------------------------------

// E4M3 byte of the value nearest to amax / (6 S); amax > 0, S > 0 finite.
__device__ __forceinline__ uint32_t scale_byte_exact(float amax, float S) {
  double r = (double)amax / (6.0 * (double)S);
  if (r >= 448.0) return 0x7Eu;
  int E;
  (void)frexp(r, &E);  // r = f 2^E, f in [0.5, 1): floor(log2 r) = E - 1
  int ep = E - 1;
  if (ep < -6) ep = -6;  // subnormal range: steps of 2^-9
  double k = rint(ldexp(r, 3 - ep));
  int b = ((ep + 6) << 3) + (int)k;  // a carry out of the mantissa bumps the exponent field
  return b > 0x7E ? 0x7Eu : (uint32_t)b;
}

// Directed conversions fp64 -> fp32 for non-negative arguments.
__device__ __forceinline__ float next_up(float f) {  // f >= 0
  uint32_t u = __float_as_uint(f);
  return (u >= 0x7f800000u) ? f : __uint_as_float(u + 1);
}
__device__ __forceinline__ float rd32(double d) {
  float f = (float)d;
  if ((double)f > d) f = __uint_as_float(__float_as_uint(f) - 1);
  return f;
}
__device__ __forceinline__ float ru32(double d) {
  float f = (float)d;
  if ((double)f < d) f = next_up(f);
  return f;
}

// Exact code magnitudes through per-block thresholds.  Boundaries between consecutive E2M1 grid
// values at t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}; a tie rounds to the even code, i.e. down at
// 0.25, 1.25, 2.5, 5 and up at 0.75, 1.75, 3.5.  U_k is the least fp32 value whose code is >= k.
__device__ __forceinline__ void codes_exact(const float v[16], float e, float S, uint32_t &w0, uint32_t &w1) {
  const double es = (double)e * (double)S;  // exact: 4 x 24 significant bits
  float U[7];
  U[0] = next_up(rd32(0.25 * es));
  U[1] = ru32(0.75 * es);
  U[2] = next_up(rd32(1.25 * es));
  U[3] = ru32(1.75 * es);
  U[4] = next_up(rd32(2.5 * es));
  U[5] = ru32(3.5 * es);
  U[6] = next_up(rd32(5.0 * es));
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float a = fabsf(v[i]);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 7; ++k) m += (a >= U[k]) ? 1u : 0u;
    m |= (__float_as_uint(v[i]) >> 28) & 8u;
    out[i >> 3] |= m << (4 * (i & 7));
  }
  w0 = out[0];
  w1 = out[1];
}

// ---- dynamic amax: per-workgroup partial maxima ------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void k_amax(const void *__restrict__ x, int64_t ld, uint32_t nblk,
                                              FastDiv bpr, float *__restrict__ partial) {
  float m = 0.0f;
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t b0 = blockIdx.x * 256u + threadIdx.x; b0 < nblk; b0 += 4 * stride) {
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // four blocks' loads in flight per thread
      const uint32_t b = (b0 + u * stride < nblk) ? b0 + u * stride : b0;
      const uint32_t row = fastdiv(b, bpr);
      const uint32_t col = b - row * bpr.d;
      BlockIn<DT>::load(x, (uint64_t)row * (uint64_t)ld + 16u * col, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[u][i]));
  }
  // workgroup reduction
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---- quantize ------------------------------------------------------------------------------------

template <int DT, bool DYNAMIC>
__global__ __launch_bounds__(256) void k_quantize(const void *__restrict__ x, int64_t ld, uint32_t nblk,
                                                  FastDiv bpr, uint8_t *__restrict__ packed,
                                                  uint8_t *__restrict__ scales, float *__restrict__ tensor_scale,
                                                  const float *__restrict__ partial, int npartial) {
  __shared__ float s_S;
  if (DYNAMIC) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < npartial; i += 256) m = fmaxf(m, partial[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      float S = amax / kDynDivisor;  // correctly rounded fp32 division
      s_S = S;
      if (blockIdx.x == 0) *tensor_scale = S;
    }
  } else {
    if (threadIdx.x == 0) s_S = *tensor_scale;
  }
  __syncthreads();
  const float S = s_S;
  const bool fast_ok = (S >= kFastSMin) && (S <= kFastSMax);
  // per-workgroup constants of the bracketing fast paths
  const double c6 = fast_ok ? 1.0 / (6.0 * (double)S) : 0.0;
  const float rlo = (float)(c6 * (1.0 - 0x1p-20)), rhi = (float)(c6 * (1.0 + 0x1p-20));
  const float invS = fast_ok ? (float)(1.0 / (double)S) : 0.0f;

  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t b0 = blockIdx.x * 256u + threadIdx.x; b0 < nblk; b0 += 2 * stride) {
    // two blocks per thread per iteration: both loads are in flight before any compute
    const uint32_t bb[2] = {b0, b0 + stride};
    float v[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t b = bb[u] < nblk ? bb[u] : b0;
      const uint32_t row = fastdiv(b, bpr);
      const uint32_t col = b - row * bpr.d;
      BlockIn<DT>::load(x, (uint64_t)row * (uint64_t)ld + 16u * col, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t b = bb[u];
      if (b >= nblk) break;
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[u][i]));

      uint32_t byte = 0, w0 = 0, w1 = 0;
      if (amax > 0.0f) {
        if (fast_ok) {
          const float ra = fminf(amax * rlo, kE4M3Max), rb = fminf(amax * rhi, kE4M3Max);
          const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, 0, false);
          byte = pk & 0xffu;
          if (byte != ((pk >> 8) & 0xffu)) byte = scale_byte_exact(amax, S);
        } else {
          byte = scale_byte_exact(amax, S);
        }
      }
      if (byte == 0) {
        // zero or flushed block: magnitude 0, sign copied
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t sgn = (__float_as_uint(v[u][i]) >> 28) & 8u;
          if (i < 8) w0 |= sgn << (4 * i);
          else w1 |= sgn << (4 * (i - 8));
        }
      } else {
        const float e = e4m3_to_f32(byte);
        bool exact = !fast_ok;
        if (fast_ok) {
          const float inv = __builtin_amdgcn_rcpf(e) * invS;
          const float ilo = inv * (1.0f - 0x1p-20f), ihi = inv * (1.0f + 0x1p-20f);
          uint32_t l0 = 0, l1 = 0, h0 = 0, h1 = 0;
#define NVFP4_ENC(J)                                                              \
  l0 = fp4_encode2<J>(l0, v[u][2 * J] * ilo, v[u][2 * J + 1] * ilo);             \
  h0 = fp4_encode2<J>(h0, v[u][2 * J] * ihi, v[u][2 * J + 1] * ihi);             \
  l1 = fp4_encode2<J>(l1, v[u][8 + 2 * J] * ilo, v[u][9 + 2 * J] * ilo);         \
  h1 = fp4_encode2<J>(h1, v[u][8 + 2 * J] * ihi, v[u][9 + 2 * J] * ihi);
          NVFP4_ENC(0)
          NVFP4_ENC(1)
          NVFP4_ENC(2)
          NVFP4_ENC(3)
#undef NVFP4_ENC
          w0 = l0;
          w1 = l1;
          exact = (l0 != h0) || (l1 != h1);
        }
        if (exact) codes_exact(v[u], e, S, w0, w1);
      }
      u32x2 o;
      o.x = w0;
      o.y = w1;
      *reinterpret_cast<u32x2 *>(packed + 8ull * b) = o;
      scales[b] = (uint8_t)byte;
    }
  }
}

// ---- launchers -------------------------------------------------------------------------------------

static int grid_for(uint32_t nblk, int cap) {
  uint32_t g = (nblk + 255u) / 256u;
  if (g < 1) g = 1;
  return (int)(g > (uint32_t)cap ? (uint32_t)cap : g);
}

hipError_t launch_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, uint8_t *packed,
                           uint8_t *scales, float *tensor_scale, bool dynamic, float *partial,
                           hipStream_t stream) {
  const uint32_t bpr_n = (uint32_t)(K / 16);
  const uint32_t nblk = (uint32_t)(M * (K / 16));
  const FastDiv bpr = make_fastdiv(bpr_n);
  const int gq = grid_for(nblk, kQuantizeMaxGrid);
  if (dynamic) {
    const int ga = grid_for(nblk, kAmaxPartials);
    if (dtype == 0) k_amax<0><<<ga, 256, 0, stream>>>(x, ld, nblk, bpr, partial);
    else k_amax<1><<<ga, 256, 0, stream>>>(x, ld, nblk, bpr, partial);
    if (dtype == 0)
      k_quantize<0, true><<<gq, 256, 0, stream>>>(x, ld, nblk, bpr, packed, scales, tensor_scale, partial, ga);
    else
      k_quantize<1, true><<<gq, 256, 0, stream>>>(x, ld, nblk, bpr, packed, scales, tensor_scale, partial, ga);
  } else {
    if (dtype == 0)
      k_quantize<0, false><<<gq, 256, 0, stream>>>(x, ld, nblk, bpr, packed, scales, tensor_scale, nullptr, 0);
    else
      k_quantize<1, false><<<gq, 256, 0, stream>>>(x, ld, nblk, bpr, packed, scales, tensor_scale, nullptr, 0);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
