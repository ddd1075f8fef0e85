/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 block-scaled 4-bit quantization and FP4-packed GEMM
 * for AMD Instinct MI355X (gfx950).
 *
 * Format [NVFP4-DiT page, Methodology section 1, Definition III.1; vllm-omni NVFP4 RFC,
 * Motivation]: every run of 16 consecutive values along K (a "block") gets one OCP E4M3FN scale
 * byte e, the whole tensor gets one fp32 scale S, and each value v becomes the 4-bit E2M1 code
 * nearest to v / (e S) (grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} with sign, ties to the even code,
 * saturating at +-6).  Readings fixed here where the pages are silent:
 *   - dynamic S = RN32(max|x| / 2688), 2688 = 6 * 448; static S is given by the caller;
 *   - e = E4M3 value nearest to max|block| / (6 S) (ties to even, saturating at 448, 0 for a
 *     block that is zero or rounds to zero; such a block's codes carry only the sign);
 *   - the code's sign bit copies the input's sign bit (so -0.0 gives code 8);
 *   - decisions are made on exact real quotients (no intermediate rounding);
 *   - element 2i of a row sits in the low nibble of byte i [NVFP4-DiT page, Methodology
 *     section 3, two FP4 values per byte].
 *
 * Canonical layouts (row-major, K contiguous):
 *   packed  uint8 [M][K/2]    scales  uint8 [M][K/16]    tensor scale  one fp32.
 * GEMM: Y[M][N] = A[M][K] * B[N][K]^T ("TN"), B being the NVFP4 weight in a prepacked layout.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers owned by the caller (any allocator); the library
 *     allocates, frees and retains nothing.  Tensor scales are device pointers too, so a
 *     dynamic activation scale feeds the GEMM without a host synchronization.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous and ordered
 *     on that stream; results are valid once the stream has reached them.
 *   - Shape, stride, alignment, dtype, mode and workspace checks run on the host before any HIP
 *     call; on failure the call returns the status and launches nothing.
 *   - After launching, a HIP error is reported as NVFP4_ERR_HIP.
 *   - Preconditions on device data (finite inputs and bias; tensor scales finite, and > 0 where
 *     the call divides by one: a STATIC quantize S and the requantizing GEMM's output S; E4M3
 *     scale bytes never 0x7F/0xFF, E8M0 scale bytes never 0xFF) are not checked by default, and
 *     results are undefined when they fail.  Debug checks (nvfp4_set_debug_checks below) scan
 *     them on the device before each call's launches.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 3

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,     /* M < 0, N < 0, K < 16, K % 16 != 0, a bad block size, or a size overflow */
  NVFP4_ERR_STRIDE = 3,    /* a leading dimension is smaller than the row it must hold */
  NVFP4_ERR_ALIGN = 4,     /* a pointer or row pitch breaks the stated alignment */
  NVFP4_ERR_DTYPE = 5,     /* unknown dtype, or a dtype the call does not accept */
  NVFP4_ERR_MODE = 6,      /* unknown mode */
  NVFP4_ERR_WORKSPACE = 7, /* workspace required but NULL or smaller than the query says */
  NVFP4_ERR_HIP = 8,       /* a HIP runtime call or kernel launch failed */
  NVFP4_ERR_DEVICE = 9,    /* the current device is not a gfx950 GPU */
  NVFP4_ERR_PRECONDITION = 10, /* debug checks on: device data the call would read breaks a precondition */
  /* Range sentinels (not statuses): they give every enum of this header the full range of int, so
     any int a caller passes -- including an invalid one, which the calls reject -- is a value of
     the type on both sides of the C / C++ boundary. */
  NVFP4_STATUS_MIN_ENUM_ = -0x7fffffff - 1,
  NVFP4_STATUS_MAX_ENUM_ = 0x7fffffff
} nvfp4_status_t;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1, NVFP4_DTYPE_MIN_ENUM_ = -0x7fffffff - 1,
               NVFP4_DTYPE_MAX_ENUM_ = 0x7fffffff } nvfp4_dtype_t;

/* W4A4: both operands NVFP4 [NVFP4-DiT page, Methodology section 3; vllm-omni RFC, Open
   Question 1].  W4A16: bf16 activations times an NVFP4 weight (weight-only quantization,
   vllm-omni RFC Open Question 1; kandinsky-5 NVFP4 pull request, Summary). */
typedef enum { NVFP4_W4A4 = 0, NVFP4_W4A16 = 1, NVFP4_MODE_MIN_ENUM_ = -0x7fffffff - 1,
               NVFP4_MODE_MAX_ENUM_ = 0x7fffffff } nvfp4_mode_t;

/* DYNAMIC: the call computes S from the input and writes it.  STATIC: the call reads a
   caller-given S (the pages' static / calibrated scale: NVFP4-DiT page, Highlights, "Static FP4";
   vllm-omni RFC, Open Question 2). */
typedef enum { NVFP4_SCALE_DYNAMIC = 0, NVFP4_SCALE_STATIC = 1, NVFP4_SCALE_MIN_ENUM_ = -0x7fffffff - 1,
               NVFP4_SCALE_MAX_ENUM_ = 0x7fffffff } nvfp4_scale_mode_t;

/* Short English text for a status; never NULL. */
const char *nvfp4_status_string(nvfp4_status_t status);

/* NVFP4_ABI_VERSION of the built library. */
int nvfp4_abi_version(void);

/* Debug checks of the preconditions on device data (off by default; diagnosis, not speed).
 *
 * When on, every call that passes its host-side checks first scans, on its stream, exactly the
 * device data it is about to read, waits for the stream, and returns NVFP4_ERR_PRECONDITION --
 * with nothing else launched and no output written -- if any value breaks the preconditions
 * stated above:
 *   quantize, fake quantize, MX quantize   every element of the logical [M][K] input finite;
 *                                          STATIC: S finite and > 0
 *   dequantize                             scale bytes not NaN; S finite
 *   prepack                                scale bytes not NaN
 *   GEMM, requantizing GEMM                W4A4: the [M][K/block] activation scale bytes not NaN,
 *                                          S_A finite; W4A16: the [M][K] bf16 activation finite;
 *                                          the prepacked weight's scale bytes not NaN, S_B finite;
 *                                          requantizing: bias finite, output S finite and > 0
 *   MX dequantize, MX GEMM                 E8M0 scale bytes not 0xFF
 * (unpack reads only bytes and is not scanned).  The wait makes every call synchronous.  A stream
 * under graph capture cannot be waited on, so captured calls skip the scans (a call on another
 * stream while a process-wide capture is running gets the runtime's refusal of its memset or
 * wait as NVFP4_ERR_HIP).  The scans use a
 * library-owned flag word per call in flight (64 of them, taken round-robin per device): more than
 * 64 calls scanning at once on one device may see each other's violations.
 *
 * The initial setting is read from the environment variable NVFP4_DEBUG when a call first needs
 * it: set and not "0" turns the checks on.  nvfp4_set_debug_checks(enable) then turns them on
 * (enable != 0) or off for every later call of the process, and returns the previous setting
 * (1 on, 0 off).  Setting it while calls on other host threads are being validated is not ordered
 * with those calls. */
int nvfp4_set_debug_checks(int enable);

/* ---------------------------------------------------------------------------------------------
 * Quantize [NVFP4-DiT page, Definition III.1; vllm-omni RFC, Motivation].
 *
 *   x            device, [M][ld_x] elements of x_dtype (fp32 or bf16), 16-byte aligned,
 *                ld_x * sizeof(elem) a multiple of 16.  Only the first K of each row are read.
 *   M, K         M >= 0; K >= 16 and K % 16 == 0.  M == 0 (an empty tensor) is valid: nothing
 *                is read or written, except that DYNAMIC writes S = 0 (the maximum over no
 *                element is taken as 0); x, packed and scales may then be NULL.
 *   packed       device, [M][K/2] bytes, written.  8-byte aligned.
 *   scales       device, [M][K/16] E4M3 bytes, written.
 *   tensor_scale device, one fp32: written by DYNAMIC, read by STATIC (finite, > 0).
 *   workspace    device scratch of nvfp4_quantize_workspace_bytes(M, K) bytes, 16-byte aligned
 *                (DYNAMIC only; may be NULL for STATIC).  Its contents need no initialization
 *                and are clobbered.
 *
 * The result is bit-identical to the definition above for every finite input.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_bytes(int64_t M, int64_t K);
nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                              uint8_t *packed, uint8_t *scales, float *tensor_scale,
                              nvfp4_scale_mode_t mode, void *workspace, size_t workspace_bytes,
                              void *stream);

/* ---------------------------------------------------------------------------------------------
 * Dequantize [NVFP4-DiT page, Definition III.1: Q = s * q]: y = RN32(q * e * S), one rounding
 * of the exact product; bf16 output is the nearest bf16 (ties to even) of that fp32 value.
 *
 *   packed, scales, tensor_scale  canonical NVFP4 tensor as written by nvfp4_quantize
 *                                 (packed 8-byte aligned).
 *   y            device, [M][ld_y] of y_dtype, 16-byte aligned, ld_y * sizeof(elem) % 16 == 0,
 *                ld_y >= K.  Columns K..ld_y-1 are not written.
 *   M == 0 is valid and touches nothing (every pointer may then be NULL).
 * ------------------------------------------------------------------------------------------- */
nvfp4_status_t nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                int64_t M, int64_t K, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                void *stream);

/* ---------------------------------------------------------------------------------------------
 * Fake quantization for quantization-aware training [NVFP4-DiT page, Methodology section 2: the
 * fake-quantize op of QAT, with a straight-through estimator for its gradient; Definition III.1].
 * Writes y = dequantize(quantize(x)) in one pass, bit-identical to nvfp4_quantize followed by
 * nvfp4_dequantize with the same S (no NVFP4 tensor is materialized).  The gradient rule (the
 * straight-through estimator) is the caller's: the Python binding's autograd function passes the
 * incoming gradient through unchanged.
 *
 *   x, x_dtype, M, K, ld_x, tensor_scale, mode, workspace   as for nvfp4_quantize.
 *   y            device, [M][ld_y] of y_dtype (fp32 or bf16), 16-byte aligned,
 *                ld_y * sizeof(elem) % 16 == 0, ld_y >= K.  Columns K..ld_y-1 are not written.
 *   M == 0 is valid (DYNAMIC still writes S = 0).
 * ------------------------------------------------------------------------------------------- */
nvfp4_status_t nvfp4_fake_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                   void *y, nvfp4_dtype_t y_dtype, int64_t ld_y, float *tensor_scale,
                                   nvfp4_scale_mode_t mode, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* ---------------------------------------------------------------------------------------------
 * Weight prepack (offline, once per weight).  Rearranges a canonical NVFP4 weight [N][K]
 * (packed [N][K/2], scales [N][K/16]) into the tile order the GEMM kernels read: N is padded
 * to a multiple of 32 and K to a multiple of 128 with zero codes and zero scales.  The layout is
 * opaque; its size is nvfp4_prepacked_bytes(N, K).  prepacked must be 16-byte aligned.  The
 * weight's tensor scale is not part of it and is passed to nvfp4_gemm separately.
 * nvfp4_unpack_weight is the exact inverse (for inspection and tests).  N == 0 is valid and
 * touches nothing (nvfp4_prepacked_bytes(0, K) == 0).
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_prepacked_bytes(int64_t N, int64_t K);
nvfp4_status_t nvfp4_prepack_weight(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K,
                                    void *prepacked, void *stream);
nvfp4_status_t nvfp4_unpack_weight(const void *prepacked, int64_t N, int64_t K, uint8_t *packed,
                                   uint8_t *scales, void *stream);

/* ---------------------------------------------------------------------------------------------
 * GEMM  Y = A * B^T  [NVFP4-DiT page, Methodology section 3: packed FP4 operands dequantized on
 * the fly, FP32 accumulation].  Operands are dequantized exactly (each q * e is exact in 16-bit
 * floating point) and multiplied on the matrix cores with fp32 accumulation; S_A * S_B is applied
 * to the fp32 accumulator before the output conversion.  Only the summation order differs from
 * the dequantize-then-matmul definition.
 *
 *   mode           NVFP4_W4A4: a = packed [M][lda/2] bytes (8-byte aligned), a_scales = [M][lda/16]
 *                  E4M3 bytes (4-byte aligned), a_tensor_scale = device fp32 S_A (as written by
 *                  nvfp4_quantize; lda == K for its output).  lda % 16 == 0, lda >= K.
 *                  NVFP4_W4A16: a = bf16 [M][lda] (lda >= K, lda * 2 % 16 == 0, 16-byte aligned);
 *                  a_scales and a_tensor_scale must be NULL.
 *   b_prepacked    weight from nvfp4_prepack_weight(N, K); b_tensor_scale its device fp32 S_B.
 *   c              device, [M][ldc] of c_dtype (fp32 or bf16), ldc >= N, base 16-byte aligned.
 *   workspace      device scratch of nvfp4_gemm_workspace_bytes_ld(mode, M, N, K, lda) bytes (may
 *                  be NULL when that is 0), 16-byte aligned; contents need no initialization.  The
 *                  activation's row pitch is part of the plan (a W4A4 lda that is not a multiple of
 *                  128, for one, selects another kernel), so the query takes it;
 *                  nvfp4_gemm_workspace_bytes(mode, M, N, K) is the same query with lda == K.  A
 *                  workspace smaller than the query for the call's own lda returns
 *                  NVFP4_ERR_WORKSPACE and launches nothing.
 *   Extents: M, N < 2^30, K < 2^30, N * K and M * N <= 2^40, M * lda <= 2^40 (else
 *   NVFP4_ERR_SHAPE; the queries return 0 for such arguments).
 *   M == 0 or N == 0 (an empty output) is valid and touches nothing; the pointers may be NULL.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_gemm_workspace_bytes(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K);
size_t nvfp4_gemm_workspace_bytes_ld(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K, int64_t lda);
nvfp4_status_t nvfp4_gemm(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales, const float *a_tensor_scale,
                          const void *b_prepacked, const float *b_tensor_scale, int64_t M, int64_t N, int64_t K,
                          int64_t lda, void *c, nvfp4_dtype_t c_dtype, int64_t ldc, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Other block sizes [NVFP4-DiT page, Methodology section 2, Algorithm 1 / Eq. 9 (a block size per
 * layer from {1, ..., 64}) and the configuration table (a fixed block size)].  block_size =
 * values per E4M3 scale byte along K, one of 16, 32, 64; K % block_size == 0; scales are then
 * [rows][K / block_size] bytes.  Everything else (tensor scale, rounding, packing, layouts,
 * alignments, errors) is as for the calls without the suffix, which are these with block_size 16.
 * A weight prepacked with any block size is read by every GEMM call the same way (its scales are
 * expanded to one byte per 16 k); a_block_size is the W4A4 activation's block size (lda must be a
 * multiple of it) and is ignored for W4A16.  nvfp4_gemm* also need a_scales 4-byte aligned.
 * nvfp4_unpack_weight_bs inverts nvfp4_prepack_weight_bs of the same block size: it returns the
 * byte stored for the first 16 k of each block, so unpacking with a block size other than the one
 * the weight was prepacked with does not recover its scales.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status_t nvfp4_quantize_bs(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                 int block_size, uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                 nvfp4_scale_mode_t mode, void *workspace, size_t workspace_bytes, void *stream);
nvfp4_status_t nvfp4_dequantize_bs(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                   int64_t M, int64_t K, int block_size, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                   void *stream);
nvfp4_status_t nvfp4_fake_quantize_bs(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                      int block_size, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                      float *tensor_scale, nvfp4_scale_mode_t mode, void *workspace,
                                      size_t workspace_bytes, void *stream);
nvfp4_status_t nvfp4_prepack_weight_bs(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K,
                                       int block_size, void *prepacked, void *stream);
nvfp4_status_t nvfp4_unpack_weight_bs(const void *prepacked, int64_t N, int64_t K, int block_size, uint8_t *packed,
                                      uint8_t *scales, void *stream);
nvfp4_status_t nvfp4_gemm_bs(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                             const float *a_tensor_scale, int a_block_size, const void *b_prepacked,
                             const float *b_tensor_scale, int64_t M, int64_t N, int64_t K, int64_t lda, void *c,
                             nvfp4_dtype_t c_dtype, int64_t ldc, void *workspace, size_t workspace_bytes,
                             void *stream);

/* ---------------------------------------------------------------------------------------------
 * Quantize without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments, checks
 * and results as nvfp4_quantize_bs, minus the workspace: the dynamic pass's partial maxima go to a
 * scratch array the library holds in device memory, 4096 bytes (NVFP4 quantize workspace) per GPU,
 * kept from the first call on that GPU until the process ends.  Every size nvfp4_quantize_bs
 * accepts fits it (its workspace query is 4096 bytes for every M, K); a call whose need exceeded
 * the scratch would return NVFP4_ERR_WORKSPACE and launch nothing.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine); the caller passes inputs and outputs.
 * All calls on one GPU share its scratch: calls that overlap on one GPU (different streams without
 * ordering between them) race and give undefined results; calls ordered on a stream do not.  No
 * scratch contents carry from one call to the next (each call writes every partial it reads).
 * STATIC mode uses no scratch.  With debug checks on (nvfp4_set_debug_checks) the call also scans
 * its input first and waits on its stream, as every call then does; the scans allocate nothing
 * either (their flag words are another static device array).
 * ------------------------------------------------------------------------------------------- */
nvfp4_status_t nvfp4_quantize_noalloc(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                      int block_size, uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                      nvfp4_scale_mode_t mode, void *stream);

/* ---------------------------------------------------------------------------------------------
 * GEMM with NVFP4 output (epilogue-fused requantization) [NVFP4-DiT page, Methodology section 3:
 * packed operands for the next W4A4 product, produced on the fly; Definition III.1 for the
 * encoding].  The product is formed exactly as in nvfp4_gemm; in fp32,
 *     y = acc * S_A * S_B  (+ bias[n] when bias != NULL)  (then act(y))
 * and y is quantized under the STATIC output tensor scale *out_tensor_scale with nvfp4_quantize's
 * rules (exact decisions on the fp32 value y), written in the canonical layout: out_packed
 * [M][N/2] bytes, out_scales [M][N/16] E4M3 bytes.  The result can feed nvfp4_gemm as the next
 * W4A4 activation (lda = N) together with out_tensor_scale.  A dynamic output scale would need the
 * whole output's maximum before the first block is encoded, so it is not offered.
 *
 *   mode, a, a_scales, a_tensor_scale, b_prepacked, b_tensor_scale, M, N, K, lda: as nvfp4_gemm.
 *   N % 16 == 0 (the output's 16-value blocks run along N).
 *   bias           NULL or device fp32 [N], 16-byte aligned.
 *   act            NVFP4_ACT_NONE, or NVFP4_ACT_GELU_TANH: 0.5 y (1 + tanh(sqrt(2/pi)(y + 0.044715 y^3)))
 *                  (the pages do not name the MLP activation; the tanh form of GELU is the one of
 *                  the DiT-family MLPs they build on).
 *   out_tensor_scale  device fp32 static S of the output (finite, > 0).
 *   out_packed     device [M][N/2], 16-byte aligned.   out_scales  device [M][N/16].
 *   y              NULL, or device fp32 [M][ld_y] (ld_y >= N, ld_y % 4 == 0, 16-byte aligned) that
 *                  also receives the fp32 values that were quantized.
 *   workspace      nvfp4_gemm_requant_workspace_bytes_ld(mode, M, N, K, lda) bytes, 16-byte aligned
 *                  (may be NULL when that is 0); nvfp4_gemm_requant_workspace_bytes(mode, M, N, K) is
 *                  the same query with lda == K.  A shorter workspace returns NVFP4_ERR_WORKSPACE.
 *   M == 0 or N == 0 is valid and touches nothing.
 * ------------------------------------------------------------------------------------------- */
typedef enum { NVFP4_ACT_NONE = 0, NVFP4_ACT_GELU_TANH = 1, NVFP4_ACT_MIN_ENUM_ = -0x7fffffff - 1,
               NVFP4_ACT_MAX_ENUM_ = 0x7fffffff } nvfp4_act_t;

size_t nvfp4_gemm_requant_workspace_bytes(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K);
size_t nvfp4_gemm_requant_workspace_bytes_ld(nvfp4_mode_t mode, int64_t M, int64_t N, int64_t K, int64_t lda);
nvfp4_status_t nvfp4_gemm_requant(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                                  const float *a_tensor_scale, const void *b_prepacked, const float *b_tensor_scale,
                                  int64_t M, int64_t N, int64_t K, int64_t lda, const float *bias, nvfp4_act_t act,
                                  const float *out_tensor_scale, uint8_t *out_packed, uint8_t *out_scales, float *y,
                                  int64_t ld_y, void *workspace, size_t workspace_bytes, void *stream);
/* The same with the W4A4 activation's block size (see the block-size calls above); the output is
   written with 16-value blocks. */
nvfp4_status_t nvfp4_gemm_requant_bs(nvfp4_mode_t mode, const void *a, const uint8_t *a_scales,
                                     const float *a_tensor_scale, int a_block_size, const void *b_prepacked,
                                     const float *b_tensor_scale, int64_t M, int64_t N, int64_t K, int64_t lda,
                                     const float *bias, nvfp4_act_t act, const float *out_tensor_scale,
                                     uint8_t *out_packed, uint8_t *out_scales, float *y, int64_t ld_y, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * MXFP4, the related microscaling format (vllm-omni RFC, Motivation; the pages do not define it,
 * the OCP microscaling definition is followed): blocks of 32 consecutive values along K share one
 * E8M0 scale byte b (X = 2^(b - 127)), X = 2^(floor(log2 amax) - 2) with b clamped to [0, 254] and
 * b = 0 for an all-zero block; each value is the E2M1 code nearest to v / X (ties to the even code,
 * clipped to +-6, sign copied); there is no tensor scale.  Codes are packed as for NVFP4 (element 2i
 * in the low nibble of byte i, [M][K/2]); scales are [M][K/32] bytes.  K >= 32, K % 32 == 0,
 * M == 0 is valid and touches nothing.
 *
 * nvfp4_mx_quantize    x as for nvfp4_quantize (fp32 or bf16, 16-byte aligned rows); packed
 *                      8-byte aligned.  Bit-identical to the definition for every finite input.
 * nvfp4_mx_dequantize  y = q * X (exact for every byte the quantizer produces); bf16 output is
 *                      the nearest bf16 of it.  y as for nvfp4_dequantize.
 * nvfp4_mx_gemm        Y = A * B^T with A [M][K] and B [N][K] both canonical MXFP4 (a, b 16-byte
 *                      aligned; a_scales, b_scales 4-byte aligned), on the block-scaled FP4 matrix
 *                      instruction: the products are exact in fp32 and accumulate in fp32, so only
 *                      the summation order differs from dequantize-then-matmul.  c as for
 *                      nvfp4_gemm (fp32 or bf16, base 16-byte aligned, ldc >= N).  N == 0 is valid.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status_t nvfp4_mx_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                 uint8_t *packed, uint8_t *scales, void *stream);
nvfp4_status_t nvfp4_mx_dequantize(const uint8_t *packed, const uint8_t *scales, int64_t M, int64_t K, void *y,
                                   nvfp4_dtype_t y_dtype, int64_t ld_y, void *stream);
nvfp4_status_t nvfp4_mx_gemm(const uint8_t *a, const uint8_t *a_scales, const uint8_t *b, const uint8_t *b_scales,
                             int64_t M, int64_t N, int64_t K, void *c, nvfp4_dtype_t c_dtype, int64_t ldc,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
