// NVFP4 dequantization for gfx950: y = RN32(q * e * S) [NVFP4-DiT page, Definition III.1,
// Q = s * q with s = e * S].  q * e is exact in fp32 (<= 2 x 4 significant bits), so the single
// multiply by S is the only rounding; bf16 output rounds that fp32 value to nearest-even
// (v_cvt_pk_bf16_f32).
//
// Lane-contiguous: a lane owns one 16-byte segment of the output (8 bf16 or 4 fp32 values), reads
// its 4 or 2 code bytes and its block's scale byte, so every wave-wide store is one contiguous 1-KB
// span and the code loads are contiguous too.  Each lane keeps four or eight segments' loads in
// flight.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {
// segments per lane: eight keep more bytes in flight on large tensors; small ones keep four, so
// that the grid still has enough waves
constexpr int kSegsSmall = 4, kSegsLarge = 8;
constexpr bool kCodesNT = true;  // code bytes are read once: streaming loads
constexpr bool kOutNT = true;    // the output is written once: streaming stores
}

template <int OUT, bool DENSE, int BLK, int U>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ packed,
                                                    const uint8_t *__restrict__ scales,
                                                    const float *__restrict__ tensor_scale, uint64_t nseg,
                                                    FastDiv bpr, void *__restrict__ y, int64_t ld_y) {
  constexpr int E = (OUT == 1) ? 8 : 4;  // values per lane segment
  using Map = Segments<E, BLK>;  // a segment's block scale is byte g / Map::kLanesPerBlock
  const float S = *tensor_scale;
  const int lane = threadIdx.x & 63;
  const uint64_t ntiles = (nseg + 64 * U - 1) / (64 * U);
  for (uint64_t t = blockIdx.x * 4ull + (threadIdx.x >> 6); t < ntiles; t += gridDim.x * 4ull) {
    uint32_t codes[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t g = t * (64 * U) + u * 64 + lane;
      g = g < nseg ? g : nseg - 1;
      if constexpr (kCodesNT)
        codes[u] = (E == 8) ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(packed + 4 * g))
                            : (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(packed + 2 * g));
      else
        codes[u] = (E == 8) ? *reinterpret_cast<const uint32_t *>(packed + 4 * g)
                            : (uint32_t) * reinterpret_cast<const uint16_t *>(packed + 2 * g);
      sb[u] = scales[g >> Map::kShift];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t g = t * (64 * U) + u * 64 + lane;
      if (g >= nseg) break;
      const float e = e4m3_to_f32(sb[u]);
      float out[E];
      const f32x2 q0 = fp4_decode2_f32<0>(codes[u]), q1 = fp4_decode2_f32<1>(codes[u]);
      out[0] = (q0.x * e) * S;  // q * e is exact; the multiply by S is the one rounding
      out[1] = (q0.y * e) * S;
      out[2] = (q1.x * e) * S;
      out[3] = (q1.y * e) * S;
      if (E == 8) {
        const f32x2 q2 = fp4_decode2_f32<2>(codes[u]), q3 = fp4_decode2_f32<3>(codes[u]);
        out[4] = (q2.x * e) * S;
        out[5] = (q2.y * e) * S;
        out[6] = (q3.x * e) * S;
        out[7] = (q3.y * e) * S;
      }
      const uint64_t off = Map::template offset<DENSE>(g, bpr, ld_y);
      u32x4 o;
      if (OUT == 0) {
        o.x = __float_as_uint(out[0]);
        o.y = __float_as_uint(out[1]);
        o.z = __float_as_uint(out[2]);
        o.w = __float_as_uint(out[3]);
        store16<kOutNT>(static_cast<float *>(y) + off, o);
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
        store16<kOutNT>(static_cast<uint16_t *>(y) + off, o);
      }
    }
  }
}

// one workgroup (four waves) per four tiles of U segments per lane, up to the cap
template <int U>
static unsigned dequantize_grid(uint64_t nseg) {
  const uint64_t tiles = (nseg + 64 * U - 1) / (64 * U);
  uint64_t g = (tiles + 3) / 4;
  if (g < 1) g = 1;
  return (unsigned)(g > (uint64_t)kDequantizeMaxGrid ? (uint64_t)kDequantizeMaxGrid : g);
}

template <int BLK, int U>
static void run_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t K,
                           uint64_t nseg, void *y, int out_dtype, int64_t ld_y, hipStream_t stream) {
  const FastDiv bpr = make_fastdiv((uint32_t)(K / BLK));
  const bool dense = (ld_y == K);
  const unsigned grid = dequantize_grid<U>(nseg);
  if (out_dtype == 0) {
    if (dense) k_dequantize<0, true, BLK, U><<<grid, 256, 0, stream>>>(packed, scales, tensor_scale, nseg, bpr, y, ld_y);
    else k_dequantize<0, false, BLK, U><<<grid, 256, 0, stream>>>(packed, scales, tensor_scale, nseg, bpr, y, ld_y);
  } else {
    if (dense) k_dequantize<1, true, BLK, U><<<grid, 256, 0, stream>>>(packed, scales, tensor_scale, nseg, bpr, y, ld_y);
    else k_dequantize<1, false, BLK, U><<<grid, 256, 0, stream>>>(packed, scales, tensor_scale, nseg, bpr, y, ld_y);
  }
}

template <int BLK>
static void run_dequantize_u(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t K,
                             uint64_t nseg, void *y, int out_dtype, int64_t ld_y, hipStream_t stream) {
  // eight segments per lane once that still gives >= 4 workgroups per CU
  if (dequantize_grid<kSegsLarge>(nseg) >= 1024)
    run_dequantize<BLK, kSegsLarge>(packed, scales, tensor_scale, K, nseg, y, out_dtype, ld_y, stream);
  else
    run_dequantize<BLK, kSegsSmall>(packed, scales, tensor_scale, K, nseg, y, out_dtype, ld_y, stream);
}

hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t M,
                             int64_t K, int blk, void *y, int out_dtype, int64_t ld_y, hipStream_t stream) {
  const uint64_t nseg = (uint64_t)M * (uint64_t)K / (out_dtype == 0 ? 4u : 8u);
  if (blk == 32) run_dequantize_u<32>(packed, scales, tensor_scale, K, nseg, y, out_dtype, ld_y, stream);
  else if (blk == 64) run_dequantize_u<64>(packed, scales, tensor_scale, K, nseg, y, out_dtype, ld_y, stream);
  else run_dequantize_u<16>(packed, scales, tensor_scale, K, nseg, y, out_dtype, ld_y, stream);
  return hipGetLastError();
}

}  // namespace nvfp4
