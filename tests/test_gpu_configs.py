"""GPU parity on every workload at its full size, and on row-strided W4A4 activations.

Quantization is compared byte for byte with the oracle on every tensor the workloads quantize:
the PixArt-style block's four activations (1 % outlier channels x20) and weights, the weight-only
variant's Laplace-tailed fp32 weights, the video-DiT Student-t x LogNormal activations and weights,
and all six sweep tensors (dynamic, and static with the x2^10 blocks), with their dequantization
bit for bit [NVFP4-DiT page, Definition III.1; vllm-omni RFC, Motivation: the two-level scale].
The PixArt block's four GEMMs and the three video-DiT GEMMs are compared on every output element.
GEMM bar: |Y_gpu - Y| <= 1e-5 sum_k |a_ik b_jk| per
element (fp32 output), plus 2^-8 |Y| of output rounding for bf16 output.

Row-strided W4A4 activations (a view of wider packed rows, lda > K, whose padding holds codes and
scale bytes that must be ignored) go through nvfp4_gemm and nvfp4_gemm_requant at block sizes 16,
32 and 64: lda = K + 128 keeps the tiled kernels, a pitch that is not a multiple of 128 runs the
generic kernel [NVFP4-DiT page, Methodology section 3: packed operands dequantized on the fly].
"""
import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
import workloads
from test_gpu_parity import DEV, Guarded, assert_quantize_exact, check_gemm, np_bf16, np_x, run_fake, say

pytestmark = pytest.mark.gpu


# ---- quantize bytes on every workload tensor ---------------------------------------------------------

def test_quantize_pixart_activations_and_weights():
    for name, x, w in workloads.pixart():
        assert_quantize_exact(x, label=f"pixart {name} activation")
        assert_quantize_exact(w, label=f"pixart {name} weight")


def test_quantize_w4a16_weights_fp32():
    for name, (w, acts) in workloads.w4a16().items():
        assert w.dtype == torch.float32
        assert_quantize_exact(w, label=f"w4a16 {name} weight (fp32, Laplace tails)")


def test_quantize_video_activations_and_weights():
    for name, x, w in workloads.video():
        assert_quantize_exact(x, label=f"video {name} activation")
        assert_quantize_exact(w, label=f"video {name} weight")


@pytest.mark.parametrize("M,K", [(4096, 12288), (32768, 1152), (32768, 3072)])
def test_quantize_sweep_remaining_shapes(M, K):
    """The sweep shapes the other tests leave out: dynamic and static (x2^10 blocks under S = 2^-8)
    quantization bit-exact, and the dynamic result dequantized to bf16 and fp32 bit for bit."""
    x = workloads.sweep(M, K)
    (p, s, S), (op, os_, oS) = assert_quantize_exact(x, label="sweep dynamic")
    say(f"[dequantize] sweep {M}x{K}")
    y32_o, y16_o = oracle.dequantize(op, os_, oS)
    g16 = nv.nvfp4_dequantize(p, s, S, torch.bfloat16)
    g32 = nv.nvfp4_dequantize(p, s, S, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(np_bf16(g16), y16_o)
    assert np.array_equal(g32.cpu().numpy().view(np.uint32), y32_o.view(np.uint32))
    del g16, g32, y32_o, y16_o
    xs = workloads.sweep(M, K, static=True)
    assert_quantize_exact(xs, static_S=workloads.SWEEP_STATIC_S, label="sweep static")


def test_quantize_sweep_largest_static_pass():
    """The largest sweep tensor's static pass: every 101st block x2^10 under S = 2^-8 (saturated 0x7E
    scales and clipped codes), at the launch shape the benchmark times."""
    xs = workloads.sweep(32768, 12288, static=True)
    (p, s, S), (op, os_, oS) = assert_quantize_exact(xs, static_S=workloads.SWEEP_STATIC_S,
                                                     label="sweep 32768x12288 static")
    assert (os_ == 0x7E).any()


# ---- GEMMs of the workloads ---------------------------------------------------------------------------

def _oracle_operands(x_cpu, w_cpu, rows=None, cols=None):
    xo, wo = np_x(x_cpu), np_x(w_cpu)
    SA, SB = oracle.tensor_scale(xo), oracle.tensor_scale(wo)
    if rows is not None:
        xo = np.ascontiguousarray(xo[rows])
    if cols is not None:
        wo = np.ascontiguousarray(wo[cols])
    ap, as_, _ = oracle.quantize(xo, S=SA)
    bp, bs, _ = oracle.quantize(wo, S=SB)
    A, _ = oracle.dequantize(ap, as_, SA)
    B, _ = oracle.dequantize(bp, bs, SB)
    return A, B, SA, SB


def _gpu_w4a4(x_cpu, w_cpu, out_dtype):
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    wp, ws, wS = nv.nvfp4_quantize(w_cpu.to(DEV))
    bp = nv.nvfp4_prepack_weight(wp, ws)
    pa, sa, Sa = nv.nvfp4_quantize(x_cpu.to(DEV))
    esz = 4 if out_dtype == torch.float32 else 2
    gy = Guarded(M * N * esz)
    out = gy.payload((M, N), out_dtype)
    nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, out_dtype, out=out)
    torch.cuda.synchronize()
    gy.check()
    return out.float().cpu().numpy(), np.float32(Sa.item()), np.float32(wS.item())


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_pixart_every_output(out_dtype):
    """All four PixArt-style block GEMMs (M = 4096) on every output element, in the launch
    configuration the benchmark times (bf16 out) and with fp32 out."""
    for name, x, w in workloads.pixart():
        M, K = x.shape
        N = w.shape[0]
        say(f"[gemm W4A4 full] pixart {name} {M}x{N}x{K} out={out_dtype}")
        Yg, Sa, Sb = _gpu_w4a4(x, w, out_dtype)
        A, B, SA, SB = _oracle_operands(x, w)
        assert Sa == SA and Sb == SB
        Y, R = oracle.gemm(A, B)
        check_gemm(Yg, Y, R, out_dtype == torch.bfloat16, f"pixart {name}")


def test_gemm_video_every_output():
    """The three video-DiT GEMMs (M = 10240) on every output element, bf16 out as the benchmark runs
    them; the oracle's fp64 product is formed 2048 rows at a time."""
    for name, x, w in workloads.video():
        M, K = x.shape
        N = w.shape[0]
        say(f"[gemm W4A4 full] video {name} {M}x{N}x{K}")
        Yg, Sa, Sb = _gpu_w4a4(x, w, torch.bfloat16)
        A, B, SA, SB = _oracle_operands(x, w)
        assert Sa == SA and Sb == SB
        for r0 in range(0, M, 2048):
            Y, R = oracle.gemm(A[r0:r0 + 2048], B)
            check_gemm(Yg[r0:r0 + 2048], Y, R, True, f"video {name} rows {r0}..{min(M, r0 + 2048) - 1}")


@pytest.mark.parametrize("static", [False, True])
def test_fake_quantize_large_tensor(static):
    """Fake quantization (bf16 out) of the 32768 x 3072 sweep tensor: large enough for the widened
    grid, where a dynamic pass reduces the amax partials once in its own kernel."""
    x = workloads.sweep(32768, 3072, static=static)
    run_fake(x, workloads.SWEEP_STATIC_S if static else None, torch.bfloat16, label="sweep 32768x3072")


# ---- row-strided W4A4 activations ---------------------------------------------------------------------

def _strided_activation(x_cpu, b, lda):
    """Quantize x on the device, then copy codes and scales into rows of lda values whose padding
    holds codes 0xF (-6) and scale bytes 0x7E (448): a view [M, K/2] / [M, K/b] with pitch lda."""
    M, K = x_cpu.shape
    pa, sa, Sa = nv.nvfp4_quantize(x_cpu.to(DEV), block_size=b)
    big_p = torch.full((M, lda // 2), 0xFF, dtype=torch.uint8, device=DEV)
    big_s = torch.full((M, lda // b), 0x7E, dtype=torch.uint8, device=DEV)
    big_p[:, : K // 2] = pa
    big_s[:, : K // b] = sa
    return big_p[:, : K // 2], big_s[:, : K // b], Sa


@pytest.mark.parametrize("M,N,K,b,pad", [
    (300, 272, 384, 16, 128),     # tiled 128 x 128, lda = K + 128
    (300, 272, 384, 16, 16),      # generic kernel (lda % 128 != 0)
    (300, 272, 1152, 32, 128),
    (300, 272, 1152, 32, 32),
    (300, 272, 1152, 64, 128),    # 64-blocks: byte positions shift with the row pitch
    (300, 272, 1152, 64, 64),
    (4096, 1152, 1152, 16, 128),  # the PixArt proj shape (128 x 192 tiles) with a padded activation
    (2100, 2304, 1152, 64, 128),  # 128 x 192 tiles, ragged rows, 64-blocks
    (512, 512, 4096, 64, 128),    # split-K plan
])
def test_gemm_w4a4_strided_activation(M, N, K, b, pad):
    lda = K + pad
    say(f"[gemm W4A4 strided] M={M} N={N} K={K} block={b} lda={lda}")
    g = torch.Generator().manual_seed(M + N + K + b + pad)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    wp, ws, wS = nv.nvfp4_quantize(w.to(DEV))
    bp = nv.nvfp4_prepack_weight(wp, ws)
    pa, sa, Sa = _strided_activation(x, b, lda)
    assert pa.stride(0) * 2 == lda and sa.stride(0) * b == lda
    assert nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K, lda) == \
        (nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K) if pad % 128 == 0 else 0)
    gy = Guarded(M * N * 4)
    out = gy.payload((M, N), torch.float32)
    nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.float32, out=out)
    torch.cuda.synchronize()
    gy.check()
    xo, wo = np_x(x), np_x(w)
    SA, SB = oracle.tensor_scale(xo), oracle.tensor_scale(wo)
    assert np.float32(Sa.item()) == SA
    ap, as_, _ = oracle.quantize(xo, S=SA, block=b)
    A, _ = oracle.dequantize(ap, as_, SA)
    bpo, bso, _ = oracle.quantize(wo, S=SB)
    B, _ = oracle.dequantize(bpo, bso, SB)
    Y, R = oracle.gemm(A, B)
    check_gemm(out.cpu().numpy(), Y, R, False, f"W4A4 strided lda={lda} block={b}")

    # the NVFP4-output form on the same strided operand: fp32 values within the GEMM bar (plus the
    # bias add) and bytes equal to the oracle's quantization of those values
    bias = (0.5 * torch.randn(N, generator=g)).to(torch.float32)
    yref = oracle.linear_epilogue(Y, bias.numpy(), 0)
    S_out = np.float32(float(np.max(np.abs(yref))) / 2688.0)
    So = torch.tensor([float(S_out)], dtype=torch.float32, device=DEV)
    need = nv.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, M, N, K, lda)
    if pad % 128 != 0:
        assert need == M * N * 4  # the generic kernel stages fp32 values in the workspace
    gp, gs, gyy = Guarded(M * N // 2), Guarded(M * N // 16), Guarded(M * N * 4)
    packed, scales, y = gp.payload((M, N // 2)), gs.payload((M, N // 16)), gyy.payload((M, N), torch.float32)
    nv.nvfp4_gemm_requant(nv.W4A4, pa, sa, Sa, bp, wS, N, K, So, bias=bias.to(DEV), packed=packed, scales=scales,
                          y=y)
    torch.cuda.synchronize()
    for gb in (gp, gs, gyy):
        gb.check()
    yg = y.cpu().numpy()
    err = np.abs(yg.astype(np.float64) - yref)
    tol = 1.2e-5 * R + 5e-7 * np.abs(yref) + 1e-30
    assert (err <= tol).all(), f"{int((err > tol).sum())} fp32 values outside tolerance"
    op, os_, _ = oracle.quantize(np.ascontiguousarray(yg), S=S_out)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(packed.cpu().numpy(), op)
    say(f"  requant strided: bytes exact, max err/R = {float(np.max(err / (R + 1e-30))):.3e}")
