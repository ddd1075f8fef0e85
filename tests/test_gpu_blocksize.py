"""GPU parity for block sizes 32 and 64 (one E4M3 scale byte per 32 or 64 values along K) against the
oracle [NVFP4-DiT page, Algorithm 1 / Eq. 9 block sizes; the configuration table's fixed block size].

Bars as for 16-value blocks: quantize, fake quantize, dequantize and prepack bit-exact; GEMM within
1e-5 sum|a b| per element (fp32 output).  The W4A4 cases mix activation and weight block sizes and
cover the planner's paths (256x256 and 128x128 tiles, split-K, the generic kernel), including
K = 1152 with 64-blocks, where the 18 scale bytes of a row leave every other row's bytes straddling
dword boundaries.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
from test_gpu_parity import DEV, Guarded, check_gemm, np_x, say

pytestmark = pytest.mark.gpu


def gpu_quantize_bs(x_cpu, b, static_S=None, ld=None):
    M, K = x_cpu.shape
    if ld is not None and ld != K:
        big = torch.full((M, ld), 1e30, dtype=x_cpu.dtype)  # padding must be ignored
        big[:, :K] = x_cpu
        xd = big.to(DEV)[:, :K]
    else:
        xd = x_cpu.to(DEV)
    gp, gs = Guarded(M * K // 2), Guarded(M * K // b)
    Sd = None if static_S is None else torch.tensor([static_S], dtype=torch.float32, device=DEV)
    p, s, S = nv.nvfp4_quantize(xd, Sd, packed=gp.payload((M, K // 2)), scales=gs.payload((M, K // b)),
                                block_size=b)
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    return p, s, S


def assert_quantize_bs_exact(x_cpu, b, static_S=None, ld=None, label=""):
    say(f"[quantize b={b}] {label} shape={tuple(x_cpu.shape)} {x_cpu.dtype} static={static_S} ld={ld}")
    p, s, S = gpu_quantize_bs(x_cpu, b, static_S, ld)
    op, os_, oS = oracle.quantize(np_x(x_cpu), S=static_S, block=b)
    assert np.float32(S.item()).view(np.uint32) == np.float32(oS).view(np.uint32)
    gs_, gp_ = s.cpu().numpy(), p.cpu().numpy()
    bad_s = np.nonzero(gs_ != os_)
    assert bad_s[0].size == 0, f"{bad_s[0].size} scale bytes differ, first at {bad_s[0][0], bad_s[1][0]}"
    bad_p = np.nonzero(gp_ != op)
    assert bad_p[0].size == 0, f"{bad_p[0].size} code bytes differ, first at {bad_p[0][0], bad_p[1][0]}"
    return p, s, S


@pytest.mark.parametrize("b", [32, 64])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_quantize_block_sizes(b, dt):
    g = torch.Generator().manual_seed(b * 3 + (dt == torch.float32))
    M, K = 300, 1152
    x = torch.randn(M, K, generator=g) * torch.exp(2 * torch.randn(M, 1, generator=g))
    x[0, :b] = 0.0
    x[1, :b] = -0.0
    x[2, 5] = 1e4  # one large value: small blocks elsewhere in row 2's first block
    x = x.to(dt)
    assert_quantize_bs_exact(x, b, label="dynamic")
    assert_quantize_bs_exact(x, b, static_S=0.0123, label="static")
    assert_quantize_bs_exact(x, b, static_S=1.1 * 2.0 ** -9, label="static, near-tie scale")
    assert_quantize_bs_exact(x, b, static_S=2.0 ** -12, label="static, saturating")
    assert_quantize_bs_exact(x, b, ld=K + 64, label="row stride")


@pytest.mark.parametrize("b", [32, 64])
def test_dequantize_and_fake_quantize_block_sizes(b):
    g = torch.Generator().manual_seed(50 + b)
    M, K = 257, 1216
    x = (torch.randn(M, K, generator=g) * 3).to(torch.bfloat16)
    p, s, S = assert_quantize_bs_exact(x, b, label="for dequantize")
    op, os_, oS = oracle.quantize(np_x(x), block=b)
    y32, y16 = oracle.dequantize(op, os_, oS)
    g32 = nv.nvfp4_dequantize(p, s, S, torch.float32)
    g16 = nv.nvfp4_dequantize(p, s, S, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(g32.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    assert np.array_equal(g16.cpu().view(torch.int16).numpy().view(np.uint16), y16)
    yf, _ = nv.nvfp4_fake_quantize(x.to(DEV), out_dtype=torch.float32, block_size=b)
    torch.cuda.synchronize()
    assert np.array_equal(yf.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    # the straight-through op with this block size
    xr = x.to(DEV).float().requires_grad_(True)
    y = nv.fake_quantize_ste(xr, None, b)
    y.sum().backward()
    assert torch.equal(xr.grad, torch.ones_like(xr))


@pytest.mark.parametrize("b", [32, 64])
def test_prepack_roundtrip_block_sizes(b):
    g = torch.Generator().manual_seed(b)
    N, K = 33, 1152
    packed = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    scales = torch.randint(0, 0x7F, (N, K // b), generator=g, dtype=torch.uint8)
    pp = nv.nvfp4_prepack_weight(packed.to(DEV), scales.to(DEV))
    up, us = nv.nvfp4_unpack_weight(pp, N, K, block_size=b)
    torch.cuda.synchronize()
    assert torch.equal(up.cpu(), packed) and torch.equal(us.cpu(), scales)


def run_w4a4_bs(M, N, K, ba, bb, sample=None):
    say(f"[gemm W4A4] M={M} N={N} K={K} A block {ba} B block {bb} sample={sample}")
    g = torch.Generator().manual_seed(M + 3 * N + 7 * K + ba + bb)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    wp, ws, wS = nv.nvfp4_quantize(w.to(DEV), block_size=bb)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    pa, sa, Sa = nv.nvfp4_quantize(x.to(DEV), block_size=ba)
    out = nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.float32)
    torch.cuda.synchronize()
    Yg = out.cpu().numpy()
    xo, wo = np_x(x), np_x(w)
    SA, SB = oracle.tensor_scale(xo), oracle.tensor_scale(wo)
    rows, cols = np.arange(M), np.arange(N)
    if sample is not None:
        rng = np.random.default_rng(M + N + K)
        rows = np.unique(rng.integers(0, M, sample[0]))
        cols = np.unique(rng.integers(0, N, sample[1]))
    ap, as_, _ = oracle.quantize(np.ascontiguousarray(xo[rows]), S=SA, block=ba)
    bp_o, bs_o, _ = oracle.quantize(np.ascontiguousarray(wo[cols]), S=SB, block=bb)
    A, _ = oracle.dequantize(ap, as_, SA)
    B, _ = oracle.dequantize(bp_o, bs_o, SB)
    Y, R = oracle.gemm(A, B)
    check_gemm(Yg[np.ix_(rows, cols)], Y, R, False, f"W4A4 bA={ba} bB={bb}")


@pytest.mark.parametrize("M,N,K,ba,bb", [
    (300, 272, 1152, 64, 64),    # 128x128 tiles; 64-blocks straddle dwords on odd rows
    (300, 272, 1152, 32, 16),
    (300, 272, 1152, 16, 64),
    (1024, 2304, 1024, 64, 32),  # 128x128 tiles, aligned 64-blocks
    (512, 512, 4096, 32, 64),    # split-K
    (64, 96, 192, 64, 64),       # generic kernel (K % 128 != 0)
    (1, 64, 256, 32, 32),        # one row
])
def test_gemm_w4a4_block_sizes(M, N, K, ba, bb):
    run_w4a4_bs(M, N, K, ba, bb)


def test_gemm_w4a4_block_sizes_256_tiles_sampled():
    """256x256 tiles (224 tiles, K = 1152) with 64-block activations and 32-block weights, on 96 x 96
    sampled outputs."""
    run_w4a4_bs(4096, 3456, 1152, 64, 32, sample=(96, 96))


@pytest.mark.parametrize("ba,bb", [(64, 32), (32, 64)])
def test_gemm_w4a4_block_sizes_128x192_tiles(ba, bb):
    """128x192 tiles (204 tiles, ragged rows) with 32- and 64-block operands, every output."""
    run_w4a4_bs(2100, 2304, 1152, ba, bb)


@pytest.mark.parametrize("M,N,K,bb", [(100, 512, 512, 64), (8, 512, 1024, 32), (1, 2048, 3072, 64),
                                      (3000, 2608, 384, 32)])  # half-chunk stages, two per CU
def test_gemm_w4a16_block_sizes(M, N, K, bb):
    say(f"[gemm W4A16] M={M} N={N} K={K} B block {bb}")
    g = torch.Generator().manual_seed(M + N + K + bb)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    wp, ws, wS = nv.nvfp4_quantize(w.to(DEV), block_size=bb)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    out = nv.nvfp4_gemm(nv.W4A16, x.to(DEV), None, None, bp, wS, N, K, torch.float32)
    torch.cuda.synchronize()
    bp_o, bs_o, SB = oracle.quantize(np_x(w), block=bb)
    B, _ = oracle.dequantize(bp_o, bs_o, SB)
    Y, R = oracle.gemm(oracle.bf16_to_f32(np_x(x)), B)
    check_gemm(out.cpu().numpy(), Y, R, False, f"W4A16 bB={bb}")


def test_requant_with_block_64_activation():
    """The NVFP4-output GEMM reading a 64-block activation: bytes equal the standalone quantizer's
    output of the same fp32 values (the requantization itself is covered by its own tests)."""
    g = torch.Generator().manual_seed(64)
    M, N, K = 512, 1024, 1152
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).to(DEV)
    wp, ws, wS = nv.nvfp4_quantize(w, block_size=32)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    pa, sa, Sa = nv.nvfp4_quantize(x, block_size=64)
    So = torch.tensor([2.0 / 2688.0], dtype=torch.float32, device=DEV)
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    ph, sh = nv.nvfp4_gemm_requant(nv.W4A4, pa, sa, Sa, bp, wS, N, K, So, act=nv.ACT_GELU_TANH, y=y)
    pq, sq, _ = nv.nvfp4_quantize(y, So)
    ref = nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ph, pq) and torch.equal(sh, sq)
    gelu = oracle.gelu_tanh(ref.cpu().numpy())
    err = np.abs(y.cpu().numpy() - gelu)
    assert np.all(err <= 1e-6 * np.abs(ref.cpu().numpy()) + 1e-30)
