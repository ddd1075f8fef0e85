"""GPU parity of the GEMM with NVFP4 output (epilogue-fused requantization) against the oracle.

Two bars, on identical seeded inputs:
  * the fp32 values that were quantized (the call's optional fp32 copy y) against the oracle's fp64
    y = dequant(A) dequant(B)^T (+ bias) (-> GELU): |y_gpu - y| <= 1.2e-5 R + 5e-7 |z| + 1e-30, with
    R = sum_k |a_ik b_jk| and z = Y + bias.  The GEMM alone is within 1e-5 R (summation order);
    GELU's slope is at most 1.13, and the second term covers the fp32 bias add and activation.
  * the NVFP4 bytes bit-exact against the oracle's quantization of those same fp32 values under the
    same static scale: both sides take every rounding decision on identical fp32 numbers.
Also: the call without the fp32 copy writes the same bytes; guard bands around every output stay
intact.  Each planner path is exercised: 128x128 tiles, 256x256 tiles, the 256/128 column
partition, split-K (the reduction pass requantizes), W4A16 tiles, W4A16 skinny rows, and the
generic kernel (K % 128 != 0).
"""
import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
from test_gpu_parity import DEV, Guarded, np_x, prepare_weight, say

pytestmark = pytest.mark.gpu


def run_requant(mode, M, N, K, bias_on, act, s_factor, seed, with_y=True):
    say(f"[requant] mode={'W4A4' if mode == nv.W4A4 else 'W4A16'} M={M} N={N} K={K} bias={bias_on} "
        f"act={act} S_out factor={s_factor}")
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    bias = (0.5 * torch.randn(N, generator=g)).to(torch.float32) if bias_on else None

    # oracle reference of the fp32 values before quantization
    bo_p, bo_s, SB = oracle.quantize(np_x(w))
    B, _ = oracle.dequantize(bo_p, bo_s, SB)
    if mode == nv.W4A4:
        SA = oracle.tensor_scale(np_x(x))
        ap, as_, _ = oracle.quantize(np_x(x), S=SA)
        A, _ = oracle.dequantize(ap, as_, SA)
    else:
        A = oracle.bf16_to_f32(np_x(x))
    Y, R = oracle.gemm(A, B)
    z = Y + (bias.numpy().astype(np.float64)[None, :] if bias_on else 0.0)
    yref = oracle.linear_epilogue(Y, bias.numpy() if bias_on else None, act)
    S_out = np.float32(max(float(np.max(np.abs(yref))), 1e-30) / 2688.0 * s_factor)

    # GPU
    bp, Sb, _ = prepare_weight(w)
    xd = x.to(DEV)
    if mode == nv.W4A4:
        pa, sa, Sa = nv.nvfp4_quantize(xd)
        assert np.float32(Sa.item()) == SA
        a_args = (pa, sa, Sa)
    else:
        a_args = (xd, None, None)
    So = torch.tensor([float(S_out)], dtype=torch.float32, device=DEV)
    gp, gs, gy = Guarded(M * N // 2), Guarded(M * N // 16), Guarded(M * N * 4)
    packed, scales, y = gp.payload((M, N // 2)), gs.payload((M, N // 16)), gy.payload((M, N), torch.float32)
    bias_d = bias.to(DEV) if bias_on else None
    nv.nvfp4_gemm_requant(mode, *a_args, bp, Sb, N, K, So, bias=bias_d, act=act, packed=packed, scales=scales,
                          y=y if with_y else None)
    torch.cuda.synchronize()
    for gb in (gp, gs, gy):
        gb.check()
    yg = y.cpu().numpy()

    # bar 1: the fp32 values against the fp64 reference
    err = np.abs(yg.astype(np.float64) - yref)
    tol = 1.2e-5 * R + 5e-7 * np.abs(z) + 1e-30
    bad = err > tol
    if bad.any():
        i = int(np.argmax(err / tol))
        raise AssertionError(f"{int(bad.sum())} of {bad.size} fp32 values outside tolerance; worst flat {i}: "
                             f"gpu {yg.flat[i]} ref {yref.flat[i]} R {R.flat[i]}")
    say(f"  fp32 values: max err/R = {float(np.max(err / (R + 1e-30))):.3e}")

    # bar 2: the NVFP4 bytes, bit-exact against the oracle's quantization of the same fp32 values
    op, os_, _ = oracle.quantize(np.ascontiguousarray(yg), S=S_out)
    gsn, gpn = scales.cpu().numpy(), packed.cpu().numpy()
    bad_s = np.nonzero(gsn != os_)
    assert bad_s[0].size == 0, f"{bad_s[0].size} scale bytes differ, first at {bad_s[0][0], bad_s[1][0]}"
    bad_p = np.nonzero(gpn != op)
    assert bad_p[0].size == 0, f"{bad_p[0].size} code bytes differ, first at {bad_p[0][0], bad_p[1][0]}"
    if s_factor > 1e6:
        assert (os_ == 0).all() and (op != 0).any()  # flushed blocks still carry the signs
    n_sat = int((os_ == 0x7E).sum())
    say(f"  NVFP4 bytes exact ({op.size} code bytes, {os_.size} scale bytes, {n_sat} saturated scales)")

    # the same call without the fp32 copy writes the same bytes
    if with_y:
        p2, s2 = nv.nvfp4_gemm_requant(mode, *a_args, bp, Sb, N, K, So, bias=bias_d, act=act)
        torch.cuda.synchronize()
        assert np.array_equal(p2.cpu().numpy(), gpn) and np.array_equal(s2.cpu().numpy(), gsn)


@pytest.mark.parametrize("M,N,K,bias_on,act,f", [
    (300, 272, 384, True, nv.ACT_GELU_TANH, 1.0),      # 128x128 tiles, ragged M
    (4096, 2304, 256, False, nv.ACT_NONE, 0.25),       # 128x192 tiles, saturating scale
    (4096, 3456, 256, False, nv.ACT_NONE, 1.0),        # 256x256 tiles (the last column half used)
    (4096, 4608, 128, True, nv.ACT_GELU_TANH, 1.0),    # 128x192 tiles, three per CU
    (4096, 5120, 128, True, nv.ACT_GELU_TANH, 1.0),    # 256x256 columns + 128x128 remainder
    (512, 512, 4096, True, nv.ACT_NONE, 3.7),          # split-K: the reduction requantizes
    (1, 64, 256, False, nv.ACT_NONE, 1.0),             # one row
    (64, 96, 48, True, nv.ACT_GELU_TANH, 1.0),         # generic kernel (K % 128 != 0)
    (300, 272, 384, False, nv.ACT_NONE, 1e7),          # every block flushed: byte 0, sign-only codes
    (512, 512, 4096, False, nv.ACT_GELU_TANH, 1e7),    # the same in the split-K reduction
])
def test_requant_w4a4(M, N, K, bias_on, act, f):
    run_requant(nv.W4A4, M, N, K, bias_on, act, f, seed=M * 31 + N * 7 + K)


@pytest.mark.parametrize("M,N,K,bias_on,act,f", [
    (100, 512, 512, False, nv.ACT_GELU_TANH, 1.0),     # W4A16 64x256 tiles
    (1500, 2608, 384, False, nv.ACT_NONE, 1.0),        # 128x256 tiles, whole-chunk stages
    (300, 1008, 2048, True, nv.ACT_GELU_TANH, 1.0),    # 64x256 tiles, K split: the reduction requantizes
    (2100, 304, 4096, False, nv.ACT_NONE, 0.25),       # 128x256 tiles, K split five ways, saturating
    (3000, 2608, 384, True, nv.ACT_GELU_TANH, 1.0),    # half-chunk stages, two workgroups per CU
    (8, 512, 1024, True, nv.ACT_GELU_TANH, 1.0),       # skinny rows, fp32 pass then requantize
    (1, 2048, 12288, True, nv.ACT_NONE, 0.5),          # skinny, one row, split K
    (33, 64, 80, False, nv.ACT_NONE, 1.0),             # generic kernel
])
def test_requant_w4a16(M, N, K, bias_on, act, f):
    run_requant(nv.W4A16, M, N, K, bias_on, act, f, seed=M * 37 + N * 11 + K)


def test_requant_feeds_next_w4a4_gemm():
    """The NVFP4 output is a valid W4A4 activation: gemm(requant(x)) equals gemm of the same bytes
    produced by quantizing the fp32 values with the standalone quantizer."""
    g = torch.Generator().manual_seed(99)
    M, K1, N1, N2 = 256, 512, 1024, 384
    x = torch.randn(M, K1, generator=g).to(torch.bfloat16).to(DEV)
    w1 = (0.02 * torch.randn(N1, K1, generator=g)).to(torch.bfloat16)
    w2 = (0.02 * torch.randn(N2, N1, generator=g)).to(torch.bfloat16)
    bp1, S1, _ = prepare_weight(w1)
    bp2, S2, _ = prepare_weight(w2)
    pa, sa, Sa = nv.nvfp4_quantize(x)
    So = torch.tensor([2.5 / 2688.0], dtype=torch.float32, device=DEV)
    y = torch.empty(M, N1, dtype=torch.float32, device=DEV)
    ph, sh = nv.nvfp4_gemm_requant(nv.W4A4, pa, sa, Sa, bp1, S1, N1, K1, So, act=nv.ACT_GELU_TANH, y=y)
    pq, sq, _ = nv.nvfp4_quantize(y, So)
    torch.cuda.synchronize()
    assert torch.equal(ph, pq) and torch.equal(sh, sq)
    out1 = nv.nvfp4_gemm(nv.W4A4, ph, sh, So, bp2, S2, N2, N1, torch.float32)
    out2 = nv.nvfp4_gemm(nv.W4A4, pq, sq, So, bp2, S2, N2, N1, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
