"""GPU parity of the MXFP4 path (32-value blocks, E8M0 scales, block-scaled FP4 matrix instruction)
against the CPU oracle: quantize and dequantize bit-exact, GEMM |Y_gpu - Y| <= 1e-5 sum_k |a b|
per element (fp32 out; bf16 out adds its rounding), as for NVFP4."""
import sys

import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np_x(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def mx_exact(x_cpu, ld=None, label=""):
    M, K = x_cpu.shape
    say(f"[mx quantize] {label} {tuple(x_cpu.shape)} {x_cpu.dtype} ld={ld}")
    if ld is not None and ld != K:
        big = torch.full((M, ld), 1e30, dtype=x_cpu.dtype)
        big[:, :K] = x_cpu
        xd = big.to(DEV)[:, :K]
    else:
        xd = x_cpu.to(DEV)
    p, s = nv.nvfp4_mx_quantize(xd)
    torch.cuda.synchronize()
    op, os_ = oracle.mx_quantize(np_x(x_cpu))
    gs, gp = s.cpu().numpy(), p.cpu().numpy()
    bad = np.nonzero(gs != os_)
    assert bad[0].size == 0, f"{bad[0].size} scale bytes differ, first at {bad[0][0], bad[1][0]}"
    bad = np.nonzero(gp != op)
    assert bad[0].size == 0, f"{bad[0].size} code bytes differ, first at {bad[0][0], bad[1][0]}"
    return p, s, op, os_


def test_mx_quantize_sweep_and_tiny():
    mx_exact(workloads.sweep(4096, 1152), label="sweep")
    mx_exact(workloads.sweep(4096, 3072, static=True), label="sweep with 2^10 outlier blocks")
    x, w = workloads.tiny()
    mx_exact(x, label="tiny X fp32")
    mx_exact(w, label="tiny W fp32")


@pytest.mark.parametrize("M,K,ld,dt,mag", [
    (1, 32, 32, torch.bfloat16, 0), (3, 64, 72, torch.bfloat16, 0), (33, 96, 100, torch.float32, 0),
    (255, 1152, 1152, torch.float32, -140), (17, 4096, 4104, torch.bfloat16, 120), (64, 320, 320, torch.float32, -120),
])
def test_mx_quantize_ragged_and_extremes(M, K, ld, dt, mag):
    g = torch.Generator().manual_seed(M + K + mag)
    x = torch.randn(M, K, generator=g, dtype=torch.float64) * torch.exp(2 * torch.randn(M, 1, generator=g, dtype=torch.float64))
    x = (x * 2.0 ** mag).to(torch.float32)
    x[0, :32] = 0.0
    if M > 1:
        x[1, :32] = -0.0
    mx_exact(x.to(dt), ld=ld, label=f"ragged x 2^{mag}")


@pytest.mark.parametrize("out_dtype,ld", [(torch.float32, 0), (torch.bfloat16, 0), (torch.float32, 8), (torch.bfloat16, 24)])
def test_mx_dequantize_exact(out_dtype, ld):
    rng = np.random.default_rng(7)
    M, K = 300, 1024
    p = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    s = rng.integers(0, 253, (M, K // 32), dtype=np.uint8)
    s[0, :3] = [0, 1, 252]
    say(f"[mx dequantize] {out_dtype} ld pad {ld}")
    out = torch.full((M, K + ld), 3.0, dtype=out_dtype, device=DEV)
    y = out[:, :K]
    nv.nvfp4_mx_dequantize(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV), out_dtype, out=y)
    torch.cuda.synchronize()
    y32, y16 = oracle.mx_dequantize(p, s)
    got = y.cpu().contiguous()
    if out_dtype == torch.float32:
        np.testing.assert_array_equal(got.view(torch.int32).numpy().view(np.uint32), y32.view(np.uint32))
    else:
        np.testing.assert_array_equal(got.view(torch.int16).numpy().view(np.uint16), y16)
    if ld:
        assert (out[:, K:] == 3.0).all()


def at_offset(t, off):
    """A copy of t whose data starts `off` bytes into a fresh allocation (alignment control)."""
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def run_mx_gemm(x_cpu, w_cpu, out_dtype, sample=None, scale_offset=0):
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    say(f"[mx gemm] M={M} N={N} K={K} out={out_dtype} sample={sample} scale offset={scale_offset}")
    a, as_ = nv.nvfp4_mx_quantize(x_cpu.to(DEV))
    b, bs = nv.nvfp4_mx_quantize(w_cpu.to(DEV))
    if scale_offset:
        as_, bs = at_offset(as_, scale_offset), at_offset(bs, scale_offset)
        assert as_.data_ptr() % 16 == scale_offset % 16
    pad = 8
    buf = torch.full((M, N + pad), 5.0, dtype=out_dtype, device=DEV)
    y = buf[:, :N]
    nv.nvfp4_mx_gemm(a, as_, b, bs, out=y)
    torch.cuda.synchronize()
    assert (buf[:, N:] == 5.0).all(), "columns past N written"
    Yg = y.float().cpu().numpy()
    oa, oas = oracle.mx_quantize(np_x(x_cpu))
    ob, obs = oracle.mx_quantize(np_x(w_cpu))
    assert np.array_equal(oa, a.cpu().numpy()) and np.array_equal(obs, bs.cpu().numpy())
    rows = np.arange(M) if sample is None else np.unique(np.random.default_rng(M + N).integers(0, M, sample[0]))
    cols = np.arange(N) if sample is None else np.unique(np.random.default_rng(N + K).integers(0, N, sample[1]))
    A, _ = oracle.mx_dequantize(np.ascontiguousarray(oa[rows]), np.ascontiguousarray(oas[rows]))
    B, _ = oracle.mx_dequantize(np.ascontiguousarray(ob[cols]), np.ascontiguousarray(obs[cols]))
    Y, R = oracle.gemm(A, B)
    G = Yg[np.ix_(rows, cols)].astype(np.float64)
    tol = 1e-5 * R + 1e-30
    if out_dtype == torch.bfloat16:
        tol = 2.0 ** -8 * np.abs(Y) + 1.01e-5 * R + 1e-30
    err = np.abs(G - Y)
    worst = float((err / tol).max())
    say(f"  max err / tolerance = {worst:.3e}")
    assert worst <= 1.0
    return y


def test_mx_gemm_tiny_full():
    x, w = workloads.tiny()
    run_mx_gemm(x, w, torch.float32)
    run_mx_gemm(x, w, torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (17, 33, 160), (300, 520, 256), (255, 100, 1152),
                                   (1000, 1000, 1280), (64, 64, 32), (513, 257, 384),
                                   (300, 520, 1024), (513, 257, 2048)])
def test_mx_gemm_ragged(M, N, K):
    """K % 512 == 0 (with 16-byte aligned scales) takes the 16-byte scale-block loads, the other K
    the 4-byte ones."""
    g = torch.Generator().manual_seed(M + 3 * N + 7 * K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    run_mx_gemm(x, w, torch.float32)


@pytest.mark.parametrize("K", [256, 512])
def test_mx_gemm_256_tiles_ragged(K):
    """Enough output for 256 x 256 tiles (17 x 17 of them, ragged on both sides), full comparison;
    the smaller shapes above run 128 x 128 tiles."""
    g = torch.Generator().manual_seed(K)
    x = torch.randn(4100, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(4130, K, generator=g)).to(torch.bfloat16)
    run_mx_gemm(x, w, torch.float32)


@pytest.mark.parametrize("K", [256, 512])
def test_mx_gemm_mixed_tiles_ragged(K):
    """17 columns of 256 x 256 tiles over 16 row tiles: one round of big tiles on the first 4096
    columns, the ragged last 200 columns as a second launch of 128 x 128 tiles; full comparison."""
    g = torch.Generator().manual_seed(3 * K)
    x = torch.randn(4096, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(4296, K, generator=g)).to(torch.bfloat16)
    run_mx_gemm(x, w, torch.bfloat16)


def test_mx_gemm_scales_4_byte_aligned():
    """Scale arrays that are 4- but not 16-byte aligned with K % 512 == 0: the 4-byte scale loads."""
    g = torch.Generator().manual_seed(4)
    x = torch.randn(300, 2048, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(520, 2048, generator=g)).to(torch.bfloat16)
    run_mx_gemm(x, w, torch.float32, scale_offset=4)


def test_mx_gemm_dit_shapes_every_output():
    """The four PixArt-style block GEMMs and the video-DiT qkv GEMM in MXFP4, every output element."""
    for name, x, w in workloads.pixart():
        run_mx_gemm(x, w, torch.bfloat16)
    name, x, w = workloads.video()[0]
    run_mx_gemm(x, w, torch.bfloat16)


def test_mx_gemm_deterministic():
    x, w = workloads.tiny()
    a = run_mx_gemm(x, w, torch.float32).cpu()
    b = run_mx_gemm(x, w, torch.float32).cpu()
    assert torch.equal(a, b)
