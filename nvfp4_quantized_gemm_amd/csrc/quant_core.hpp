// Exact NVFP4 encoding of one lane's values, shared by the quantize kernels and the GEMM epilogue
// that writes NVFP4 (gfx950).  The rounding rules and the exactness argument are those of the
// quantizer [NVFP4-DiT page, Methodology section 1, Definition III.1; vllm-omni NVFP4 RFC,
// Motivation]: block scale = E4M3 value nearest to amax / (6 S), element code = E2M1 value nearest
// to v / (e S), both decided on the exact real quotients, ties to even, saturating.
#pragma once
#include "common.hpp"

namespace nvfp4 {

// Per-tensor-scale constants of the bracketing fast paths.
struct QuantConsts {
  float S;          // tensor scale
  float rlo, rhi;   // RN32(c (1 -/+ 2^-20)) with c = 1 / (6 S): bracket amax / (6 S)
  float invS;       // RN32(1 / S)
  bool fast_ok;     // S inside the window where the brackets are valid
  bool ties_only;   // S a power of two and bf16 inputs: an ambiguous bracket is an exact tie
};

__device__ __forceinline__ QuantConsts make_quant_consts(float S, bool bf16_input) {
  QuantConsts qc;
  qc.S = S;
  qc.fast_ok = (S >= kFastSMin) && (S <= kFastSMax);
  const double c6 = qc.fast_ok ? 1.0 / (6.0 * (double)S) : 0.0;
  qc.rlo = (float)(c6 * (1.0 - 0x1p-20));
  qc.rhi = (float)(c6 * (1.0 + 0x1p-20));
  qc.invS = qc.fast_ok ? (float)(1.0 / (double)S) : 0.0f;
  qc.ties_only = bf16_input && qc.fast_ok && ((__float_as_uint(S) & 0x007fffffu) == 0u);
  return qc;
}

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
// Returns the n codes of v (n <= 8), value i in nibble i.
template <int N>
__device__ __forceinline__ uint32_t codes_exact(const float *v, float e, float S) {
  const double es = (double)e * (double)S;  // exact: 4 x 24 significant bits
  float U[7];
  U[0] = next_up(rd32(0.25 * es));
  U[1] = ru32(0.75 * es);
  U[2] = next_up(rd32(1.25 * es));
  U[3] = ru32(1.75 * es);
  U[4] = next_up(rd32(2.5 * es));
  U[5] = ru32(3.5 * es);
  U[6] = next_up(rd32(5.0 * es));
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float a = fabsf(v[i]);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 7; ++k) m += (a >= U[k]) ? 1u : 0u;
    m |= (__float_as_uint(v[i]) >> 28) & 8u;
    out |= m << (4 * i);
  }
  return out;
}

// Codes of the n = 4 or 8 values of one lane under block scale byte `byte` (nonzero) and tensor
// scale S: bracketing fast path, exact thresholds when the bracket is ambiguous or S is extreme.
//
// ties_only: S is a power of two and the input is bf16.  Then every value and every boundary
// t e S has at most 8 significant bits at the same scale, so a value that is not exactly on a
// boundary differs from it by at least 2^-8 relative, far outside the 2^-19 bracket: an
// ambiguous bracket is an exact tie, whose code is the even one of the two adjacent bracketing
// codes (ties to even).  That choice is made for all nibbles at once with integer operations.
//
// kFast: the caller has checked qc.fast_ok (the check then leaves the hot loop).
template <int N, bool kFast = false>
__device__ __forceinline__ uint32_t encode_values(const float *v, uint32_t byte, const QuantConsts &qc) {
  const float e = e4m3_to_f32(byte);
  const float S = qc.S;
  if (kFast || qc.fast_ok) {
    const float inv = __builtin_amdgcn_rcpf(e) * qc.invS;
    const float ilo = inv * (1.0f - 0x1p-20f), ihi = inv * (1.0f + 0x1p-20f);
    uint32_t lo = 0, hi = 0;
    lo = fp4_encode2<0>(lo, v[0] * ilo, v[1] * ilo);
    hi = fp4_encode2<0>(hi, v[0] * ihi, v[1] * ihi);
    lo = fp4_encode2<1>(lo, v[2] * ilo, v[3] * ilo);
    hi = fp4_encode2<1>(hi, v[2] * ihi, v[3] * ihi);
    if (N == 8) {
      lo = fp4_encode2<2>(lo, v[4] * ilo, v[5] * ilo);
      hi = fp4_encode2<2>(hi, v[4] * ihi, v[5] * ihi);
      lo = fp4_encode2<3>(lo, v[6] * ilo, v[7] * ilo);
      hi = fp4_encode2<3>(hi, v[6] * ihi, v[7] * ihi);
    }
    if (lo == hi) return lo;
    if (qc.ties_only) {
      const uint32_t amb = lo ^ hi;
      uint32_t d = amb | (amb >> 1);
      d |= d >> 2;                                   // bit 4i set iff nibble i differs
      const uint32_t pick = d & lo & 0x11111111u;     // differing nibbles whose lower code is odd
      const uint32_t m = pick * 15u;                  // widen to whole nibbles (no carries)
      return (lo & ~m) | (hi & m);
    }
    // A differing nibble has adjacent magnitudes m (lo) and m + 1 (hi) and the same sign: the
    // bracket is ~2^-19 wide and consecutive boundaries are >= 40 % apart.  Decide |v| against
    // the boundary t_m e S between them, exactly in fp64.
    const double es = (double)e * (double)S;  // exact: 4 + 24 significant bits
    uint32_t out = lo;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t a = (lo >> (4 * i)) & 15u, b = (hi >> (4 * i)) & 15u;
      if (a != b) {
        const uint32_t m = a & 7u;
        const double t = (m < 4u) ? 0.25 + 0.5 * (double)m : (m == 4u ? 2.5 : (m == 5u ? 3.5 : 5.0));
        const double bound = t * es;  // exact: <= 3 + 4 + 24 significant bits
        const double x = fabs((double)v[i]);
        const uint32_t mag = (x > bound) ? m + 1u : (x < bound ? m : ((m & 1u) ? m + 1u : m));
        out = (out & ~(15u << (4 * i))) | (((a & 8u) | mag) << (4 * i));
      }
    }
    return out;
  }
  return codes_exact<N>(v, e, S);
}

// E4M3 byte of the block maximum amax (>= 0) under S: bracketing fast path, exact fallback.
// kFast: the caller has checked qc.fast_ok.
template <bool kFast = false>
__device__ __forceinline__ uint32_t block_byte(float amax, const QuantConsts &qc) {
  if (!(amax > 0.0f)) return 0u;
  const float S = qc.S;
  if (kFast || qc.fast_ok) {
    const float ra = fminf(amax * qc.rlo, kE4M3Max), rb = fminf(amax * qc.rhi, kE4M3Max);
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, 0, false);
    const uint32_t b0 = pk & 0xffu, b1 = (pk >> 8) & 0xffu;
    if (b0 == b1) return b0;
    if (b1 == b0 + 1u) {
      // the ratio amax / (6 S) lies within ~2^-19 of the midpoint of two adjacent E4M3 values:
      // compare amax with 6 * midpoint * S, exact in fp64 (<= 8 + 24 significant bits)
      const double mid = 0.5 * ((double)e4m3_to_f32(b0) + (double)e4m3_to_f32(b1));
      const double bound = 6.0 * mid * (double)S;
      const double a = (double)amax;
      return (a > bound) ? b1 : (a < bound ? b0 : ((b0 & 1u) ? b1 : b0));
    }
  }
  return scale_byte_exact(amax, S);
}

// ---- branch-free fast paths (the caller settles flagged lanes with the exact functions above) ----

// Scale byte of a block from the bracket alone; `amb` is set when the two bracketing bytes differ
// (or S is outside the bracket's window), and the returned byte is then not to be used.
__device__ __forceinline__ uint32_t block_byte_fast(float amax, const QuantConsts &qc, bool &amb) {
  const float ra = fminf(amax * qc.rlo, kE4M3Max), rb = fminf(amax * qc.rhi, kE4M3Max);
  const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, 0, false);
  const uint32_t b0 = pk & 0xffu, b1 = (pk >> 8) & 0xffu;
  amb = (b0 != b1) || !qc.fast_ok;
  return b0;  // amax == 0 gives 0 * rlo = 0, byte 0
}

// Codes of 8 values (nibble i = value i) from the bracket alone, for the block's reciprocal bracket
// (ilo, ihi); a zero byte passes ilo = ihi = 0, which yields the sign-only codes of a flushed
// block.  `amb` is set when the two bracketing code words differ.
__device__ __forceinline__ uint32_t encode8_bracket(const float *v, float ilo, float ihi, bool &amb) {
  uint32_t lo = 0, hi = 0;
  lo = fp4_encode2<0>(lo, v[0] * ilo, v[1] * ilo);
  hi = fp4_encode2<0>(hi, v[0] * ihi, v[1] * ihi);
  lo = fp4_encode2<1>(lo, v[2] * ilo, v[3] * ilo);
  hi = fp4_encode2<1>(hi, v[2] * ihi, v[3] * ihi);
  lo = fp4_encode2<2>(lo, v[4] * ilo, v[5] * ilo);
  hi = fp4_encode2<2>(hi, v[4] * ihi, v[5] * ihi);
  lo = fp4_encode2<3>(lo, v[6] * ilo, v[7] * ilo);
  hi = fp4_encode2<3>(hi, v[6] * ihi, v[7] * ihi);
  amb = (lo != hi);
  return lo;
}

}  // namespace nvfp4
