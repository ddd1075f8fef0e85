// Weight prepack: canonical NVFP4 [N][K] -> the tile order read by the GEMM kernels.
//
// The GEMM feeds v_mfma_f32_32x32x16_{f16,bf16}: lane l of a wave supplies 8 consecutive k of
// column l % 32 for k-half l / 32.  A "unit" covers 32 columns x 128 k.  Inside a unit, lane
// l = c + 32 h owns the 64 codes k in [64 h, 64 h + 64) of column c (32 bytes, natural order:
// MFMA step s uses its dword s), stored as two 16-byte parts so that a wave's 16-byte reads are
// contiguous:
//   codes   [N/32][K/128][part 2][lane 64][16 B]      2048 B per unit
//   scales  [N/32][K/128][lane 64][4 B]               256 B per unit (16-k groups 4h..4h+3 of the lane)
// with the scale region following the code region.  N pads to 32, K to 128, with zero codes and
// zero scale bytes (zero scale makes padded k contribute exactly 0).  A weight quantized with
// BLK = 32 or 64 values per scale byte is expanded to one byte per 16 k (each byte repeated over
// its block), so the GEMM reads the same layout whatever the weight's block size.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

__global__ __launch_bounds__(256) void k_prepack(const uint8_t *__restrict__ packed, const uint8_t *__restrict__ scales,
                                                 int64_t N, int64_t K, int blk, int64_t Kc, uint64_t nlanes,
                                                 uint8_t *__restrict__ out, uint64_t scale_region) {
  for (uint64_t t = blockIdx.x * 256ull + threadIdx.x; t < nlanes; t += gridDim.x * 256ull) {
    const uint64_t unit = t >> 6;
    const int lane = (int)(t & 63);
    const int64_t nu = (int64_t)(unit / (uint64_t)Kc), kc = (int64_t)(unit % (uint64_t)Kc);
    const int64_t n = nu * 32 + (lane & 31);
    const int h = lane >> 5;
    // codes: bytes [kc*64 + 32h, +32) of row n, split into two 16-byte parts
    for (int p = 0; p < 2; ++p) {
      uint8_t buf[16];
      const int64_t kbyte0 = kc * 64 + 32 * h + 16 * p;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t kb = kbyte0 + i;
        buf[i] = (n < N && kb < K / 2) ? packed[n * (K / 2) + kb] : (uint8_t)0;
      }
      u32x4 v;
      v.x = buf[0] | (buf[1] << 8) | (buf[2] << 16) | ((uint32_t)buf[3] << 24);
      v.y = buf[4] | (buf[5] << 8) | (buf[6] << 16) | ((uint32_t)buf[7] << 24);
      v.z = buf[8] | (buf[9] << 8) | (buf[10] << 16) | ((uint32_t)buf[11] << 24);
      v.w = buf[12] | (buf[13] << 8) | (buf[14] << 16) | ((uint32_t)buf[15] << 24);
      *reinterpret_cast<u32x4 *>(out + unit * 2048 + (uint64_t)p * 1024 + (uint64_t)lane * 16) = v;
    }
    uint32_t sw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k16 = (kc * 8 + 4 * h + j) * 16;  // first k of the lane's j-th 16-k group
      const uint32_t s = (n < N && k16 < K) ? scales[n * (K / blk) + k16 / blk] : 0u;
      sw |= s << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(out + scale_region + unit * 256 + (uint64_t)lane * 4) = sw;
  }
}

__global__ __launch_bounds__(256) void k_unpack(const uint8_t *__restrict__ in, int64_t N, int64_t K, int blk,
                                                int64_t Kc, uint64_t nlanes, uint64_t scale_region,
                                                uint8_t *__restrict__ packed, uint8_t *__restrict__ scales) {
  for (uint64_t t = blockIdx.x * 256ull + threadIdx.x; t < nlanes; t += gridDim.x * 256ull) {
    const uint64_t unit = t >> 6;
    const int lane = (int)(t & 63);
    const int64_t nu = (int64_t)(unit / (uint64_t)Kc), kc = (int64_t)(unit % (uint64_t)Kc);
    const int64_t n = nu * 32 + (lane & 31);
    const int h = lane >> 5;
    if (n >= N) continue;
    for (int p = 0; p < 2; ++p) {
      const uint8_t *src = in + unit * 2048 + (uint64_t)p * 1024 + (uint64_t)lane * 16;
      const int64_t kbyte0 = kc * 64 + 32 * h + 16 * p;
      for (int i = 0; i < 16; ++i)
        if (kbyte0 + i < K / 2) packed[n * (K / 2) + kbyte0 + i] = src[i];
    }
    const uint8_t *ss = in + scale_region + unit * 256 + (uint64_t)lane * 4;
    for (int j = 0; j < 4; ++j) {
      const int64_t k16 = (kc * 8 + 4 * h + j) * 16;  // the first 16-k group of a block holds its byte
      if (k16 < K && k16 % blk == 0) scales[n * (K / blk) + k16 / blk] = ss[j];
    }
  }
}

hipError_t launch_prepack(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K, int blk, void *out,
                          hipStream_t stream) {
  const int64_t Nu = (N + 31) / 32, Kc = (K + 127) / 128;
  const uint64_t nlanes = (uint64_t)Nu * (uint64_t)Kc * 64ull;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  uint64_t g = (nlanes + 255) / 256;
  if (g > 65536) g = 65536;
  k_prepack<<<(unsigned)g, 256, 0, stream>>>(packed, scales, N, K, blk, Kc, nlanes, static_cast<uint8_t *>(out),
                                             scale_region);
  return hipGetLastError();
}

hipError_t launch_unpack(const void *in, int64_t N, int64_t K, int blk, uint8_t *packed, uint8_t *scales,
                         hipStream_t stream) {
  const int64_t Nu = (N + 31) / 32, Kc = (K + 127) / 128;
  const uint64_t nlanes = (uint64_t)Nu * (uint64_t)Kc * 64ull;
  const uint64_t scale_region = (uint64_t)Nu * (uint64_t)Kc * 2048ull;
  uint64_t g = (nlanes + 255) / 256;
  if (g > 65536) g = 65536;
  k_unpack<<<(unsigned)g, 256, 0, stream>>>(static_cast<const uint8_t *>(in), N, K, blk, Kc, nlanes, scale_region,
                                            packed, scales);
  return hipGetLastError();
}

}  // namespace nvfp4
