// NVFP4 quantization kernels for gfx950.
//
// Definition [NVFP4-DiT page, Methodology section 1, Definition III.1; vllm-omni NVFP4 RFC,
// Motivation]: per 16-value block an E4M3 scale e = nearest E4M3 to amax / (6 S) (ties to even,
// saturating at 448), per value the E2M1 code nearest to v / (e S) (ties to the even code,
// saturating at +-6), sign bit copied from v, two codes per byte, low nibble first.  Decisions are
// taken on the exact real quotients.
//
// Data flow: lane-contiguous.  A lane owns one 16-byte segment of the input (8 bf16 or 4 fp32
// values), so each wave-wide load is one contiguous 1-KB span; the 2 (bf16) or 4 (fp32) lanes of a
// 16-value block combine their maxima with cross-lane swaps, every lane derives the block's scale
// byte and encodes its own values, lanes store their 4 (bf16) or 2 (fp32) code bytes contiguously
// and the first lane of each block stores the scale byte.  Each lane keeps four segments' loads in
// flight (two for inputs small enough for the caches); a large input is read with streaming
// (non-temporal) loads, its last use.  Dynamic mode runs k_amax first (same mapping,
// per-workgroup partial maxima, no atomics, deterministic); every quantize workgroup reduces those
// partials itself and derives S = RN32(amax / 2688), or, on a large tensor, one workgroup does that
// once (k_tensor_scale) and a widened grid encodes.
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
//    when the two bracketing codes agree that code is the exact one.  When they disagree (a value
//    within ~2^-19 of a decision boundary, e.g. an exact tie) the bracket holds exactly one
//    boundary, between the two adjacent candidate codes, and one exact fp64 comparison of |v|
//    with that boundary t e S (<= 3 + 4 + 24 significant bits, exact) picks the code, ties to the
//    even one.  The block scale byte is settled the same way between its two candidate bytes.
//    (Scales whose mantissa is a ratio of small integers, e.g. 1.1 * 2^k, make such near-ties
//    common, so this path must be cheap.)  Outside the bracket's range of S a full exact path
//    runs: seven per-block fp32 thresholds U_k from the exact fp64 boundaries by directed
//    rounding, code = #{k : |v| >= U_k}.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "quant_core.hpp"

namespace nvfp4 {

// Segments in flight per lane: four for streamed (large) inputs; two for inputs read through the
// caches, whose launches are latency-bound and gain from twice the workgroups (PixArt block step
// 0.2082 -> 0.2054 ms; four stay better on the 805 MB tensor: 325 against 335 us).
template <bool NT>
constexpr int segs_per_lane() { return NT ? 4 : 2; }
// Streaming (non-temporal) accesses: a large input is read with them by both passes (faster from
// HBM, also when the encode pass re-reads it); an input of at most kCachedInput bytes is read with
// ordinary loads, so that the encode pass finds what the amax pass read in the last-level cache
// (9.4 MB: 9.7 -> 9.5 us; 37.7 MB followed by its GEMM: 86.6 -> 83.4 us; 63 MB alone: 30.8 ->
// 32.1 us; 805 MB: 322 -> 357 us, so not there).  Fake quantization always streams.  The NVFP4 output is stored normally so that
// the GEMM that reads it next finds it in the caches; the fake-quantization output is streamed.
constexpr uint64_t kCachedInput = 48ull << 20;
constexpr bool kOutNT = false;
constexpr bool kFakeOutNT = true;

// Fake quantization output: the lane's E codes dequantized exactly as the dequantize kernel does,
// y = RN32((q * e) * S) with q * e exact, then bf16 (nearest, ties to even) for YT = 1.
template <int E, int YT>
__device__ __forceinline__ void store_fake(uint32_t codes, uint32_t byte, float S, void *y, uint64_t off) {
  const float e = e4m3_to_f32(byte);
  float out[E];
  const f32x2 q0 = fp4_decode2_f32<0>(codes), q1 = fp4_decode2_f32<1>(codes);
  out[0] = (q0.x * e) * S;
  out[1] = (q0.y * e) * S;
  out[2] = (q1.x * e) * S;
  out[3] = (q1.y * e) * S;
  if (E == 8) {
    const f32x2 q2 = fp4_decode2_f32<2>(codes), q3 = fp4_decode2_f32<3>(codes);
    out[4] = (q2.x * e) * S;
    out[5] = (q2.y * e) * S;
    out[6] = (q3.x * e) * S;
    out[7] = (q3.y * e) * S;
  }
  if (YT == 0) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<float *>(y) + off);
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const u32x4 o = {__float_as_uint(out[4 * h]), __float_as_uint(out[4 * h + 1]), __float_as_uint(out[4 * h + 2]),
                       __float_as_uint(out[4 * h + 3])};
      store16<kFakeOutNT>(dst + h, o);
    }
  } else {
    uint32_t p[E / 2];
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const bf16x2 hh = {(__bf16)out[2 * j], (__bf16)out[2 * j + 1]};
      p[j] = __builtin_bit_cast(uint32_t, hh);
    }
    uint16_t *dst = static_cast<uint16_t *>(y) + off;
    if (E == 8) {
      const u32x4 o = {p[0], p[1], p[2], p[3]};
      store16<kFakeOutNT>(dst, o);
    } else {
      const u32x2 o = {p[0], p[1]};
      *reinterpret_cast<u32x2 *>(dst) = o;
    }
  }
}

// ---- dynamic amax: per-workgroup partial maxima ------------------------------------------------------

template <int DT, bool DENSE, bool NT>
__global__ __launch_bounds__(256) void k_amax(const void *__restrict__ x, int64_t ld, uint64_t nseg,
                                              FastDiv bpr, float *__restrict__ partial) {
  using In = SegIn<DT>;
  using Map = Segments<In::kElems>;
  constexpr int U = segs_per_lane<NT>();
  const int lane = threadIdx.x & 63;
  const uint64_t ntiles = (nseg + 64 * U - 1) / (64 * U);
  float m = 0.0f;
  for (uint64_t t = blockIdx.x * 4ull + (threadIdx.x >> 6); t < ntiles; t += gridDim.x * 4ull) {
    float v[U][In::kElems];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t g = t * (64 * U) + u * 64 + lane;
      g = g < nseg ? g : nseg - 1;  // a repeated segment does not change the maximum
      In::unpack(In::template raw<NT>(x, Map::template offset<DENSE>(g, bpr, ld)), v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < In::kElems; ++i) m = fmaxf(m, fabsf(v[u][i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[4];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// This thread's share of the maximum of the npartial (<= kAmaxPartials) partial maxima: all of its
// loads are issued before the first comparison.
__device__ __forceinline__ float partial_max(const float *__restrict__ partial, int npartial) {
  static_assert(kAmaxPartials % 256 == 0, "partials per thread");
  float v[kAmaxPartials / 256];
#pragma unroll
  for (int j = 0; j < kAmaxPartials / 256; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < npartial ? partial[i] : 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kAmaxPartials / 256; ++j) m = fmaxf(m, v[j]);
  return m;
}

// Tensor scale S = RN32(amax / 2688) from the amax pass's partial maxima, in one workgroup.
__global__ __launch_bounds__(256) void k_tensor_scale(const float *__restrict__ partial, int npartial,
                                                      float *__restrict__ tensor_scale) {
  float m = partial_max(partial, npartial);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) *tensor_scale = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / kDynDivisor;
}

// ---- quantize ------------------------------------------------------------------------------------

// YT < 0: write the NVFP4 tensor (packed codes + scale bytes).  YT = 0 / 1: fake quantization,
// write dequantize(quantize(x)) as fp32 / bf16 into y [.][ld_y] instead (one pass, same values as
// the two calls).
template <int DT, bool DYNAMIC, bool DENSE, int YT, int BLK, bool NT>
__device__ __forceinline__ void quantize_body(const void *__restrict__ x, int64_t ld, uint64_t nseg, FastDiv bpr,
                                              uint8_t *__restrict__ packed, uint8_t *__restrict__ scales,
                                              float *__restrict__ tensor_scale, const float *__restrict__ partial,
                                              int npartial, void *__restrict__ y, int64_t ld_y) {
  using In = SegIn<DT>;
  constexpr int E = In::kElems;
  using Map = Segments<E, BLK>;  // a block of BLK values spans Map::kLanesPerBlock adjacent lanes
  constexpr int U = segs_per_lane<NT>();
  // the first tile's input loads are independent of S: issue them before the scale reduction
  const int lane = threadIdx.x & 63;
  const uint64_t ntiles = (nseg + 64 * U - 1) / (64 * U);
  const uint64_t tstride = gridDim.x * 4ull;
  auto fetch = [&](uint64_t t, u32x4 *r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t g = t * (64 * U) + u * 64 + lane;
      g = g < nseg ? g : nseg - 1;
      r[u] = In::template raw<NT>(x, Map::template offset<DENSE>(g, bpr, ld));
    }
  };
  uint64_t t = blockIdx.x * 4ull + (threadIdx.x >> 6);
  u32x4 nxt[U];
  if (t < ntiles) fetch(t, nxt);

  __shared__ float s_S;
  if (DYNAMIC) {
    float m = partial_max(partial, npartial);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      const float S = amax / kDynDivisor;  // correctly rounded fp32 division
      s_S = S;
      if (blockIdx.x == 0) *tensor_scale = S;
    }
  } else {
    if (threadIdx.x == 0) s_S = *tensor_scale;
  }
  __syncthreads();
  const float S = s_S;
  const QuantConsts qc = make_quant_consts(S, DT == 1);

  // block maximum over the block's lanes (nseg is a multiple of the lanes per block, so a block's
  // lanes are all in range or all out of range)
  auto block_amax = [&](const float (&v)[E]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(v[i]));
    return group_max<Map::kLanesPerBlock>(amax);
  };
  // scale byte and codes of one segment of a block with maximum amax (kFast: qc.fast_ok holds)
  auto encode_block = [&](auto fast_tag, const float (&v)[E], float amax, uint32_t &byte) {
    constexpr bool kFast = decltype(fast_tag)::value;
    byte = block_byte<kFast>(amax, qc);
    uint32_t codes = 0;
    if (byte == 0) {  // zero or flushed block: magnitude 0, sign copied
#pragma unroll
      for (int i = 0; i < E; ++i) codes |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * i);
    } else {
      codes = encode_values<E, kFast>(v, byte, qc);
    }
    return codes;
  };

  // Dense NVFP4 output: the tiles wholly inside the tensor run with one base address per tile and
  // constant offsets for the lane's segments, and two register sets take turns holding the next
  // tile's loads (no copies).  The one partial tile, if any, goes through the general loop below.
  // This loop runs for S inside the brackets' window (it then carries no per-block test of the
  // window); an extreme S takes the general loop throughout.
  if constexpr (DENSE && YT < 0) {
    const uint64_t nfull = nseg / (64 * U);
    auto dense_loop = [&](auto fast_tag) {
      const u32x4 *xs = static_cast<const u32x4 *>(x) + lane;
      auto fetch_full = [&](uint64_t tt, u32x4 (&r)[U]) {
        const u32x4 *p = xs + tt * (64 * U);
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = load16<NT>(p + u * 64);
      };
      auto run_tile = [&](const u32x4 (&r)[U], uint64_t tt) {
        const uint64_t g0 = tt * (64 * U) + lane;  // segment of u = 0; u adds 64
        uint8_t *pk = packed + (E / 2) * g0;
        uint8_t *sc = scales + (g0 >> Map::kShift);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[E];
          In::unpack(r[u], v);
          uint32_t byte;
          const uint32_t codes = encode_block(fast_tag, v, block_amax(v), byte);
          if (E == 8) *reinterpret_cast<uint32_t *>(pk + u * 64 * 4) = codes;
          else *reinterpret_cast<uint16_t *>(pk + u * 64 * 2) = (uint16_t)codes;
          if ((lane & (Map::kLanesPerBlock - 1)) == 0) sc[u * (64 >> Map::kShift)] = (uint8_t)byte;
        }
      };
      u32x4 alt[U];
      for (;;) {
        if (t + tstride < nfull) fetch_full(t + tstride, alt);
        run_tile(nxt, t);
        t += tstride;
        if (t >= nfull) break;
        if (t + tstride < nfull) fetch_full(t + tstride, nxt);
        run_tile(alt, t);
        t += tstride;
        if (t >= nfull) break;
      }
      if (t < ntiles) fetch(t, nxt);
    };
    if (t < nfull && qc.fast_ok) dense_loop(std::true_type{});
  }

  // encodes one segment (its E values already unpacked) as segment g
  auto encode_seg = [&](const float (&v)[E], uint64_t g) {
    const float amax = block_amax(v);
    if (g >= nseg) return;
    uint32_t byte;
    const uint32_t codes = encode_block(std::false_type{}, v, amax, byte);
    if (YT < 0) {
      if constexpr (kOutNT) {
        if (E == 8) __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t *>(packed + 4 * g));
        else __builtin_nontemporal_store((uint16_t)codes, reinterpret_cast<uint16_t *>(packed + 2 * g));
        if ((lane & (Map::kLanesPerBlock - 1)) == 0)
          __builtin_nontemporal_store((uint8_t)byte, scales + (g >> Map::kShift));
      } else {
        if (E == 8) *reinterpret_cast<uint32_t *>(packed + 4 * g) = codes;
        else *reinterpret_cast<uint16_t *>(packed + 2 * g) = (uint16_t)codes;
        if ((lane & (Map::kLanesPerBlock - 1)) == 0) scales[g >> Map::kShift] = (uint8_t)byte;
      }
    } else {
      store_fake<E, YT>(codes, byte, S, y, Map::template offset<DENSE>(g, bpr, ld_y));
    }
  };

  for (; t < ntiles; t += tstride) {
    // the next tile's loads are issued before this tile is encoded
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    if (t + tstride < ntiles) fetch(t + tstride, nxt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[E];
      In::unpack(cur[u], v);
      encode_seg(v, t * (64 * U) + u * 64 + lane);
    }
  }
}

// The NVFP4-output kernel is held to 96 VGPRs, five waves per SIMD: on a 805 MB bf16 tensor this
// moved the static pass from 190 to 175 us.  Fake quantization keeps the compiler's choice (under
// the same cap it spills inside its loop).
template <int DT, bool DYNAMIC, bool DENSE, int BLK, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void k_quantize(
    const void *__restrict__ x, int64_t ld, uint64_t nseg, FastDiv bpr, uint8_t *__restrict__ packed,
    uint8_t *__restrict__ scales, float *__restrict__ tensor_scale, const float *__restrict__ partial, int npartial) {
  quantize_body<DT, DYNAMIC, DENSE, -1, BLK, NT>(x, ld, nseg, bpr, packed, scales, tensor_scale, partial, npartial,
                                                 nullptr, 0);
}

template <int DT, bool DYNAMIC, bool DENSE, int YT, int BLK>
__global__ __launch_bounds__(256) void k_fake_quantize(const void *__restrict__ x, int64_t ld, uint64_t nseg,
                                                       FastDiv bpr, float *__restrict__ tensor_scale,
                                                       const float *__restrict__ partial, int npartial,
                                                       void *__restrict__ y, int64_t ld_y) {
  quantize_body<DT, DYNAMIC, DENSE, YT, BLK, true>(x, ld, nseg, bpr, nullptr, nullptr, tensor_scale, partial,
                                                   npartial, y, ld_y);
}

// ---- launchers -------------------------------------------------------------------------------------

static int grid_for(uint64_t nseg, int cap, int segs) {
  const uint64_t tiles = (nseg + 64 * segs - 1) / (64 * segs);
  uint64_t g = (tiles + 3) / 4;  // four waves per workgroup
  if (g < 1) g = 1;
  return (int)(g > (uint64_t)cap ? (uint64_t)cap : g);
}

// bpr16 / bpr: blocks of 16 / of BLK values per row (the amax pass maps segments with 16-blocks)
template <int DT, bool DENSE, int YT, int BLK>
static void run_quantize(const void *x, int64_t ld, uint64_t nseg, FastDiv bpr16, FastDiv bpr, uint8_t *packed,
                         uint8_t *scales, float *tensor_scale, bool dynamic, float *partial, void *y, int64_t ld_y,
                         hipStream_t stream) {
  // Large tensors widen the encode grid.  A dynamic pass then reduces the amax partials once
  // (k_tensor_scale, one workgroup) and runs the static kernel, which reads S; on smaller tensors
  // every encode workgroup of the resident grid reduces the partials itself (one launch fewer).
  auto run = [&](auto nt_tag) {
    constexpr bool NT = decltype(nt_tag)::value;
    constexpr int U = segs_per_lane<NT>();
    const bool wide = grid_for(nseg, 1 << 30, U) > kQuantizeWideFrom;
    const int gq = grid_for(nseg, wide ? kQuantizeWideGrid : kQuantizeMaxGrid, U);
    const int ga = dynamic ? grid_for(nseg, kAmaxPartials, U) : 0;
    if (dynamic) {
      k_amax<DT, DENSE, NT><<<ga, 256, 0, stream>>>(x, ld, nseg, bpr16, partial);
      if (wide) k_tensor_scale<<<1, 256, 0, stream>>>(partial, ga, tensor_scale);
    }
    const bool dyn_kernel = dynamic && !wide;
    if constexpr (YT < 0) {
      if (dyn_kernel)
        k_quantize<DT, true, DENSE, BLK, NT><<<gq, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales, tensor_scale,
                                                                     partial, ga);
      else
        k_quantize<DT, false, DENSE, BLK, NT><<<gq, 256, 0, stream>>>(x, ld, nseg, bpr, packed, scales, tensor_scale,
                                                                      nullptr, 0);
    } else {
      if (dyn_kernel)
        k_fake_quantize<DT, true, DENSE, YT, BLK><<<gq, 256, 0, stream>>>(x, ld, nseg, bpr, tensor_scale, partial, ga,
                                                                          y, ld_y);
      else
        k_fake_quantize<DT, false, DENSE, YT, BLK><<<gq, 256, 0, stream>>>(x, ld, nseg, bpr, tensor_scale, nullptr, 0,
                                                                           y, ld_y);
    }
  };
  if constexpr (YT >= 0) {
    run(std::true_type{});
  } else {
    if (nseg * 16ull > kCachedInput) run(std::true_type{});
    else run(std::false_type{});
  }
}

template <int YT, int BLK>
static void dispatch_dt(const void *x, int dtype, int64_t K, int64_t ld, uint64_t nseg, FastDiv bpr16,
                        uint8_t *packed, uint8_t *scales, float *tensor_scale, bool dynamic, float *partial, void *y,
                        int64_t ld_y, hipStream_t stream) {
  const FastDiv bpr = make_fastdiv((uint32_t)(K / BLK));
  const bool dense = (ld == K) && (YT < 0 || ld_y == K);
  if (dtype == 0) {
    if (dense)
      run_quantize<0, true, YT, BLK>(x, ld, nseg, bpr16, bpr, packed, scales, tensor_scale, dynamic, partial, y, ld_y,
                                     stream);
    else
      run_quantize<0, false, YT, BLK>(x, ld, nseg, bpr16, bpr, packed, scales, tensor_scale, dynamic, partial, y,
                                      ld_y, stream);
  } else {
    if (dense)
      run_quantize<1, true, YT, BLK>(x, ld, nseg, bpr16, bpr, packed, scales, tensor_scale, dynamic, partial, y, ld_y,
                                     stream);
    else
      run_quantize<1, false, YT, BLK>(x, ld, nseg, bpr16, bpr, packed, scales, tensor_scale, dynamic, partial, y,
                                      ld_y, stream);
  }
}

template <int YT>
static void dispatch_quantize(const void *x, int dtype, int64_t K, int64_t ld, int blk, uint8_t *packed,
                              uint8_t *scales, float *tensor_scale, bool dynamic, float *partial, void *y,
                              int64_t ld_y, int64_t M, hipStream_t stream) {
  const FastDiv bpr16 = make_fastdiv((uint32_t)(K / 16));
  const uint64_t nseg = (uint64_t)M * (uint64_t)K / (dtype == 0 ? 4u : 8u);
  if (blk == 32)
    dispatch_dt<YT, 32>(x, dtype, K, ld, nseg, bpr16, packed, scales, tensor_scale, dynamic, partial, y, ld_y, stream);
  else if (blk == 64)
    dispatch_dt<YT, 64>(x, dtype, K, ld, nseg, bpr16, packed, scales, tensor_scale, dynamic, partial, y, ld_y, stream);
  else
    dispatch_dt<YT, 16>(x, dtype, K, ld, nseg, bpr16, packed, scales, tensor_scale, dynamic, partial, y, ld_y, stream);
}

hipError_t launch_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, int blk, uint8_t *packed,
                           uint8_t *scales, float *tensor_scale, bool dynamic, float *partial,
                           hipStream_t stream) {
  dispatch_quantize<-1>(x, dtype, K, ld, blk, packed, scales, tensor_scale, dynamic, partial, nullptr, 0, M, stream);
  return hipGetLastError();
}

// ---- library-owned scratch (the no-allocation quantize entry point) ----------------------------------
// The dynamic pass's per-workgroup partial maxima, for callers that cannot allocate a workspace.
// Each GPU holds its own copy of this array from the first use until the process ends; every call on
// a GPU shares it (each call writes every partial it reads before reading it, so nothing needs
// clearing, and calls that overlap on one GPU race).  In host code the array's name is only a
// stand-in: its device address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) float scratch[kAmaxPartials];
static_assert(sizeof(scratch) == kQuantizeScratchBytes, "scratch size");
static std::atomic<float *> scratch_addr[kMaxDevices];

hipError_t quantize_scratch(float **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float *p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void *q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (q == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float *>(q);
    scratch_addr[dev].store(p, std::memory_order_release);  // concurrent first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_fake_quantize(const void *x, int dtype, int64_t M, int64_t K, int64_t ld, int blk, void *y,
                                int y_dtype, int64_t ld_y, float *tensor_scale, bool dynamic, float *partial,
                                hipStream_t stream) {
  if (y_dtype == 0)
    dispatch_quantize<0>(x, dtype, K, ld, blk, nullptr, nullptr, tensor_scale, dynamic, partial, y, ld_y, M, stream);
  else
    dispatch_quantize<1>(x, dtype, K, ld, blk, nullptr, nullptr, tensor_scale, dynamic, partial, y, ld_y, M, stream);
  return hipGetLastError();
}

}  // namespace nvfp4
