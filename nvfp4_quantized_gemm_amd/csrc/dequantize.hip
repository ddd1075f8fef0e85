// NVFP4 dequantization for gfx950: y = RN32(q * e * S) [NVFP4-DiT page, Definition III.1,
// Q = s * q with s = e * S].  q * e is exact in fp32 (<= 2 x 4 significant bits), so the single
// multiply by S is the only rounding; bf16 output rounds that fp32 value to nearest-even
// (v_cvt_pk_bf16_f32).  One thread owns one 16-value block: 8 B of codes + 1 scale byte in,
// 64 B (fp32) or 32 B (bf16) out.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

template <int OUT>
__device__ __forceinline__ void dequant_block(u32x2 w, uint32_t byte, float S, void *y, uint64_t off) {
  const float e = e4m3_to_f32(byte);
  const f32x2 q[8] = {fp4_decode2_f32<0>(w.x), fp4_decode2_f32<1>(w.x), fp4_decode2_f32<2>(w.x),
                      fp4_decode2_f32<3>(w.x), fp4_decode2_f32<0>(w.y), fp4_decode2_f32<1>(w.y),
                      fp4_decode2_f32<2>(w.y), fp4_decode2_f32<3>(w.y)};
  float out[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    out[2 * j] = (q[j].x * e) * S;  // q * e is exact; the multiply by S is the one rounding
    out[2 * j + 1] = (q[j].y * e) * S;
  }
  if (OUT == 0) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<float *>(y) + off);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x4 o;
      o.x = __float_as_uint(out[4 * q4]);
      o.y = __float_as_uint(out[4 * q4 + 1]);
      o.z = __float_as_uint(out[4 * q4 + 2]);
      o.w = __float_as_uint(out[4 * q4 + 3]);
      __builtin_nontemporal_store(o, dst + q4);
    }
  } else {
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + off);
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      uint32_t p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x2 h = {(__bf16)out[8 * q4 + 2 * t], (__bf16)out[8 * q4 + 2 * t + 1]};
        p[t] = __builtin_bit_cast(uint32_t, h);
      }
      u32x4 o;
      o.x = p[0];
      o.y = p[1];
      o.z = p[2];
      o.w = p[3];
      __builtin_nontemporal_store(o, dst + q4);
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ packed,
                                                    const uint8_t *__restrict__ scales,
                                                    const float *__restrict__ tensor_scale, uint32_t nblk,
                                                    FastDiv bpr, void *__restrict__ y, int64_t ld_y) {
  const float S = *tensor_scale;
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t b0 = blockIdx.x * 256u + threadIdx.x; b0 < nblk; b0 += 4 * stride) {
    u32x2 w[4];
    uint32_t sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // four blocks' loads in flight per thread
      const uint32_t b = (b0 + u * stride < nblk) ? b0 + u * stride : b0;
      w[u] = *reinterpret_cast<const u32x2 *>(packed + 8ull * b);
      sb[u] = scales[b];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t b = b0 + u * stride;
      if (b >= nblk) break;
      const uint32_t row = fastdiv(b, bpr);
      const uint32_t col = b - row * bpr.d;
      dequant_block<OUT>(w[u], sb[u], S, y, (uint64_t)row * (uint64_t)ld_y + 16ull * col);
    }
  }
}

hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t M,
                             int64_t K, void *y, int out_dtype, int64_t ld_y, hipStream_t stream) {
  const uint32_t nblk = (uint32_t)(M * (K / 16));
  const FastDiv bpr = make_fastdiv((uint32_t)(K / 16));
  uint32_t g = (nblk + 255u) / 256u;
  if (g > (uint32_t)kDequantizeMaxGrid) g = kDequantizeMaxGrid;
  if (out_dtype == 0)
    k_dequantize<0><<<g, 256, 0, stream>>>(packed, scales, tensor_scale, nblk, bpr, y, ld_y);
  else
    k_dequantize<1><<<g, 256, 0, stream>>>(packed, scales, tensor_scale, nblk, bpr, y, ld_y);
  return hipGetLastError();
}

}  // namespace nvfp4
