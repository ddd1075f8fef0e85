"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on identical seeded inputs.

Bars: quantize, dequantize and prepack bit-exact (codes, scale bytes, tensor scale, output bit
patterns including the sign of zero); GEMM |Y_gpu - Y| <= 1e-5 * sum_k |a_ik b_jk| per element for
fp32 output (only the summation order differs), plus the output rounding 2^-8 |Y| for bf16 output.
Every output buffer sits between canary guard bands that must stay untouched.
"""
import math
import sys

import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
GUARD = 256
CANARY = 0xA5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---- helpers ------------------------------------------------------------------------------------

def np_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np_x(t: torch.Tensor) -> np.ndarray:
    """Oracle view of an input tensor: float32 stays float32, bf16 becomes its bit patterns."""
    if t.dtype == torch.bfloat16:
        return np_bf16(t)
    return t.detach().cpu().contiguous().numpy()


class Guarded:
    """A device byte buffer with canary bands around the payload."""

    def __init__(self, nbytes: int):
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=DEV)

    def payload(self, shape, dtype=torch.uint8):
        return self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def check(self):
        b = self.buf.cpu().numpy()
        assert (b[:GUARD] == CANARY).all() and (b[GUARD + self.n:] == CANARY).all(), "guard band overwritten"


def gpu_quantize(x_cpu: torch.Tensor, static_S=None, ld=None):
    M, K = x_cpu.shape
    if ld is not None and ld != K:
        big = torch.zeros((M, ld), dtype=x_cpu.dtype)
        big[:, :K] = x_cpu
        big[:, K:] = 1e30 if x_cpu.dtype == torch.float32 else 1e30  # must be ignored
        xd = big.to(DEV)[:, :K]
    else:
        xd = x_cpu.to(DEV)
    gp, gs = Guarded(M * K // 2), Guarded(M * K // 16)
    Sd = None if static_S is None else torch.tensor([static_S], dtype=torch.float32, device=DEV)
    p, s, S = nv.nvfp4_quantize(xd, Sd, packed=gp.payload((M, K // 2)), scales=gs.payload((M, K // 16)))
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    return p.cpu().numpy(), s.cpu().numpy(), np.float32(S.item()), (p, s, S)


def assert_quantize_exact(x_cpu, static_S=None, ld=None, label=""):
    say(f"[quantize] {label} shape={tuple(x_cpu.shape)} dtype={x_cpu.dtype} static={static_S} ld={ld}")
    gp_, gs_, gS, dev = gpu_quantize(x_cpu, static_S, ld)
    op, os_, oS = oracle.quantize(np_x(x_cpu), S=static_S)
    assert np.float32(gS).view(np.uint32) == np.float32(oS).view(np.uint32), (gS, oS)
    bad_s = np.nonzero(gs_ != os_)
    assert bad_s[0].size == 0, f"{bad_s[0].size} scale bytes differ, first at {bad_s[0][0], bad_s[1][0]}"
    bad_p = np.nonzero(gp_ != op)
    assert bad_p[0].size == 0, f"{bad_p[0].size} code bytes differ, first at {bad_p[0][0], bad_p[1][0]}"
    return dev, (op, os_, oS)


# ---- quantize -------------------------------------------------------------------------------------

def test_quantize_tiny_fp32_dynamic():
    x, w = workloads.tiny()
    assert_quantize_exact(x, label="tiny X")
    assert_quantize_exact(w, label="tiny W")


@pytest.mark.parametrize("M,K", [(4096, 1152), (4096, 3072)])
def test_quantize_sweep_dynamic_and_static(M, K):
    x = workloads.sweep(M, K)
    assert_quantize_exact(x, label="sweep dynamic")
    xs = workloads.sweep(M, K, static=True)
    assert_quantize_exact(xs, static_S=workloads.SWEEP_STATIC_S, label="sweep static")


@pytest.mark.parametrize("M,K,ld,dt", [
    (1, 16, 16, torch.bfloat16), (1, 16, 16, torch.float32), (17, 48, 56, torch.bfloat16),
    (255, 1168, 1168, torch.bfloat16), (3, 4096, 4104, torch.bfloat16), (33, 80, 84, torch.float32),
    (1000, 272, 272, torch.float32),
])
def test_quantize_ragged_shapes_and_strides(M, K, ld, dt):
    g = torch.Generator().manual_seed(M * 7 + K)
    x = torch.randn(M, K, generator=g) * torch.exp(3 * torch.randn(M, 1, generator=g))
    x[0, :16] = 0.0
    if M > 1:
        x[1, :16] = -0.0
    x = x.to(dt)
    assert_quantize_exact(x, ld=ld, label="ragged dynamic")
    assert_quantize_exact(x, static_S=0.0123, ld=ld, label="ragged static")


def test_quantize_all_zero_tensor():
    x = torch.zeros(8, 64, dtype=torch.bfloat16)
    x[3, 5] = -0.0
    dev, (op, os_, oS) = assert_quantize_exact(x, label="all zero")
    assert oS == 0.0 and (os_ == 0).all()


def test_quantize_extreme_static_scales():
    """Static S far outside the fast-path window exercises the exact threshold path everywhere."""
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(64, 128, generator=g) * 1e-30).to(torch.float32)
    assert_quantize_exact(x, static_S=2.0 ** -120, label="tiny S")
    x = (torch.randn(64, 128, generator=g) * 1e30).to(torch.float32)
    assert_quantize_exact(x, static_S=2.0 ** 110, label="huge S")


@pytest.mark.parametrize("S", [1.1 * 2.0 ** -9, 1.5 * 2.0 ** -9, 1.25 * 2.0 ** -9, 1.75 * 2.0 ** -10,
                               2.0 ** -8 / 3.0, 2.0 ** -9 / 7.0, 1.0 / 2688.0])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_quantize_near_tie_scales(S, dt):
    """Static scales whose mantissa is a ratio of small integers put many values (and block maxima)
    exactly on, or within an fp32 rounding of, a decision boundary t e S or an E4M3 midpoint; every
    such value is decided by the exact two-candidate comparison.  Inputs: random values plus
    dyadic multiples of the block scale (on-boundary candidates)."""
    g = torch.Generator().manual_seed(int(S * 2.0 ** 40) % 100003)
    M, K = 512, 2048
    x = torch.randn(M, K, generator=g) * 0.5
    # every third row: small integers times 2^-k, so t e S boundaries are hit exactly or nearly
    ints = torch.randint(-48, 49, (M // 3, K), generator=g).to(torch.float32)
    x[::3][: M // 3] = ints * 2.0 ** -7
    x = x.to(dt)
    assert_quantize_exact(x, static_S=float(np.float32(S)), label=f"near-tie S={S:.6g}")


def test_quantize_sweep_full_size_largest():
    """Largest sweep tensor (32768 x 12288 bf16, 403M values), dynamic, full comparison.  Then, at
    the same size (the launch shapes the benchmark times: grid-stride over a capped grid, eight
    segments per dequantize lane): static quantization with the dynamic S gives the same bytes,
    dequantization to bf16 equals the oracle's bit for bit, and fake quantization (static and
    dynamic) equals that dequantization."""
    x = workloads.sweep(32768, 12288)
    (p, s, S), (op, os_, oS) = assert_quantize_exact(x, label="sweep 32768x12288")
    xd = x.to(DEV)
    say("[static quantize, dequantize, fake quantize] 32768x12288")
    p2, s2, _ = nv.nvfp4_quantize(xd, S.clone())
    assert torch.equal(p2, p) and torch.equal(s2, s)
    del p2, s2
    y = nv.nvfp4_dequantize(p, s, S, torch.bfloat16)
    _, y16_o = oracle.dequantize(op, os_, oS)
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero(yb != y16_o)
    assert bad[0].size == 0, f"{bad[0].size} dequantized values differ, first at {bad[0][0], bad[1][0]}"
    del yb, y16_o
    fs, _ = nv.nvfp4_fake_quantize(xd, S.clone())
    assert torch.equal(fs.view(torch.int16), y.view(torch.int16))
    del fs
    fd, Sd = nv.nvfp4_fake_quantize(xd)
    assert torch.equal(Sd, S)
    assert torch.equal(fd.view(torch.int16), y.view(torch.int16))


def test_quantize_deterministic():
    x = workloads.sweep(4096, 1152)
    a = gpu_quantize(x)
    b = gpu_quantize(x)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all() and a[2] == b[2]


# ---- dequantize -------------------------------------------------------------------------------------

# (8191, 3072): eight segments per lane, with a ragged last tile
@pytest.mark.parametrize("M,K", [(4096, 1152), (17, 48), (8191, 3072)])
def test_dequantize_exact_bits(M, K):
    x = workloads.sweep(M, K) if M == 4096 else torch.randn(M, K, generator=torch.Generator().manual_seed(3)).to(
        torch.bfloat16)
    say(f"[dequantize] {M}x{K}")
    (p, s, S), (op, os_, oS) = assert_quantize_exact(x, label="for dequant")
    y32_o, y16_o = oracle.dequantize(op, os_, oS)
    for dt, ref in ((torch.float32, y32_o.view(np.uint32)), (torch.bfloat16, y16_o)):
        esz = 4 if dt == torch.float32 else 2
        ld = K + (16 // esz)  # padded rows: the pad must stay untouched
        gy = Guarded(M * ld * esz)
        out = gy.payload((M, ld), dt)
        out_view = out[:, :K]
        nv.nvfp4_dequantize(p, s, S, dt, out=out_view)
        torch.cuda.synchronize()
        gy.check()
        raw = gy.buf[GUARD:GUARD + M * ld * esz].cpu().numpy()
        if dt == torch.float32:
            bits = raw.view(np.uint32).reshape(M, ld)
        else:
            bits = raw.view(np.uint16).reshape(M, ld)
        np.testing.assert_array_equal(bits[:, :K], ref)
        pad = raw.reshape(M, ld * esz)[:, K * esz:]
        assert (pad == CANARY).all(), "row padding written"


def test_requantize_roundtrip_on_gpu():
    """Quantize -> dequantize (fp32) -> quantize with the same static S reproduces bytes 0 and >= 3."""
    x = workloads.sweep(4096, 1152)
    (p, s, S), (op, os_, oS) = assert_quantize_exact(x, label="roundtrip")
    y = nv.nvfp4_dequantize(p, s, S, torch.float32)
    p2, s2, _ = nv.nvfp4_quantize(y, S)
    s_np, s2_np = s.cpu().numpy().ravel(), s2.cpu().numpy().ravel()
    keep = (s_np == 0) | (s_np >= 3)
    np.testing.assert_array_equal(s2_np[keep], s_np[keep])
    np.testing.assert_array_equal(p2.cpu().numpy().reshape(-1, 8)[keep], p.cpu().numpy().reshape(-1, 8)[keep])


# ---- prepack --------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(32, 128), (33, 144), (1152, 1152), (100, 16), (3072, 12288)])
def test_prepack_roundtrip(N, K):
    g = torch.Generator().manual_seed(N + K)
    packed = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    scales = torch.randint(0, 0x7F, (N, K // 16), generator=g, dtype=torch.uint8)
    pp = nv.nvfp4_prepack_weight(packed.to(DEV), scales.to(DEV))
    assert pp.numel() == nv.nvfp4_prepacked_bytes(N, K)
    up, us = nv.nvfp4_unpack_weight(pp, N, K)
    torch.cuda.synchronize()
    assert torch.equal(up.cpu(), packed) and torch.equal(us.cpu(), scales)


# ---- GEMM -------------------------------------------------------------------------------------------

def check_gemm(Yg: np.ndarray, Y: np.ndarray, R: np.ndarray, bf16_out: bool, label: str):
    err = np.abs(Yg.astype(np.float64) - Y)
    tol = 1e-5 * R
    if bf16_out:
        tol = 2.0 ** -8 * np.abs(Y) + 1.01e-5 * R
    tol = tol + 1e-30  # all-zero rows
    bad = err > tol
    if bad.any():
        i = np.argmax(err / tol)
        raise AssertionError(f"{label}: {int(bad.sum())} of {bad.size} outside tolerance; worst "
                             f"flat index {i}: gpu {Yg.flat[i]} ref {Y.flat[i]} R {R.flat[i]}")
    say(f"  {label}: max err/R = {float(np.max(err / (R + 1e-30))):.3e}")


def prepare_weight(w_cpu: torch.Tensor):
    p, s, S, _ = gpu_quantize(w_cpu)
    pd, sd, Sd = [torch.from_numpy(a).to(DEV) for a in (p, s)] + [torch.tensor([S], device=DEV)]
    bp = nv.nvfp4_prepack_weight(pd, sd)
    return bp, Sd, (p, s, S)


def run_w4a4(x_cpu, w_cpu, out_dtype, sample=None):
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    say(f"[gemm W4A4] M={M} N={N} K={K} out={out_dtype} sample={sample}")
    bp, Sb, (wp, ws, wS) = prepare_weight(w_cpu)
    xd = x_cpu.to(DEV)
    pa, sa, Sa = nv.nvfp4_quantize(xd)
    esz = 4 if out_dtype == torch.float32 else 2
    gy = Guarded(M * N * esz)
    out = gy.payload((M, N), out_dtype)
    nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, Sb, N, K, out_dtype, out=out)
    torch.cuda.synchronize()
    gy.check()
    Yg = out.float().cpu().numpy()
    # oracle: its own quantization of both operands, dequantize, fp64 matmul
    xo = np_x(x_cpu)
    SA = oracle.tensor_scale(xo)
    assert SA == np.float32(Sa.item())
    if sample is None:
        ap, as_, _ = oracle.quantize(xo, S=SA)
        A, _ = oracle.dequantize(ap, as_, SA)
        bo_p, bo_s, SB = oracle.quantize(np_x(w_cpu))
        B, _ = oracle.dequantize(bo_p, bo_s, SB)
        Y, R = oracle.gemm(A, B)
        check_gemm(Yg, Y, R, out_dtype == torch.bfloat16, f"W4A4 {M}x{N}x{K}")
    else:
        rng = np.random.default_rng(M + N + K)
        rows = np.unique(rng.integers(0, M, sample[0]))
        cols = np.unique(rng.integers(0, N, sample[1]))
        ap, as_, _ = oracle.quantize(np.ascontiguousarray(xo[rows]), S=SA)
        A, _ = oracle.dequantize(ap, as_, SA)
        SB = oracle.tensor_scale(np_x(w_cpu))
        bo_p, bo_s, _ = oracle.quantize(np.ascontiguousarray(np_x(w_cpu)[cols]), S=SB)
        B, _ = oracle.dequantize(bo_p, bo_s, SB)
        Y, R = oracle.gemm(A, B)
        check_gemm(Yg[np.ix_(rows, cols)], Y, R, out_dtype == torch.bfloat16, f"W4A4 {M}x{N}x{K} sampled")
    return out


def test_gemm_w4a4_tiny_full():
    x, w = workloads.tiny()
    run_w4a4(x, w, torch.float32)
    run_w4a4(x, w, torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (17, 33, 144), (255, 100, 1152), (300, 520, 256),
                                   (64, 64, 16), (129, 257, 384), (1000, 1000, 1280)])
def test_gemm_w4a4_ragged(M, N, K):
    g = torch.Generator().manual_seed(M + 3 * N + 7 * K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    run_w4a4(x, w, torch.float32)


@pytest.mark.parametrize("M,N,K,split", [
    (512, 512, 4096, True),      # 16 tiles of 128 x 128, K split
    (4096, 1024, 4096, False),   # 256 tiles of 128 x 128, one per CU
    (2048, 4096, 1024, False),   # 512 tiles of 128 x 128, two per CU
    (4096, 1664, 2048, True),    # 416 small tiles, 288 of 128 x 192: 256 x 256 tiles, K split two ways
    (3072, 1408, 2048, False),   # 264 small tiles: 192 tiles of 128 x 192 (the last column 64 wide)
])
def test_gemm_w4a4_planner_paths(M, N, K, split):
    """One shape per plan of the W4A4 planner below one round of 256 x 256 tiles (sampled outputs);
    the workspace query says whether the plan splits K."""
    assert (nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K) > 0) == split
    g = torch.Generator().manual_seed(M + N + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    run_w4a4(x, w, torch.bfloat16, sample=(64, 64))


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (2100, 2302, 1152, torch.bfloat16),  # ragged rows and columns; rows not 16-byte aligned (N % 8 != 0)
    (2048, 2304, 1152, torch.float32),   # 192 tiles, one per CU
    (4096, 2304, 1152, torch.float32),   # 384 tiles: two workgroups on half of the CUs
])
def test_gemm_w4a4_128x192_tiles(M, N, K, out_dtype):
    """Every output of the W4A4 GEMM on shapes the planner gives 128 x 192 tiles (two 96-column wave
    sub-tiles, stored as a 64- and a 32-column piece; two B scale units past the tile fetched and
    unused)."""
    assert nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K) == 0
    g = torch.Generator().manual_seed(M + 5 * N + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    run_w4a4(x, w, out_dtype)


@pytest.mark.parametrize("M,N,K", [
    (256, 1152, 2304),    # 18 tiles of 128 x 128, 18 chunks: split six ways, three chunks each
    (256, 3072, 4608),    # 48 tiles, 36 chunks: split four ways
    (512, 1152, 4608),    # 36 tiles: split four ways (9 chunks each)
    (1024, 1152, 4608),   # 72 tiles: split three ways
    (300, 1000, 2304),    # ragged M and N with a K split (18 tiles of 128 x 128)
])
def test_gemm_w4a4_small_m_split_plans(M, N, K):
    """Every output of the W4A4 GEMM at small-M shapes whose 128 x 128 plan splits K over the idle
    CUs (the splits differ in their chunk counts when K does not divide evenly)."""
    g = torch.Generator().manual_seed(M + 2 * N + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    run_w4a4(x, w, torch.float32)


def test_gemm_w4a4_pixart_full_size_sampled():
    for name, x, w in workloads.pixart():
        run_w4a4(x, w, torch.bfloat16, sample=(96, 96))


def test_gemm_w4a4_video_full_size_sampled():
    for name, x, w in workloads.video():
        run_w4a4(x, w, torch.bfloat16, sample=(48, 48))


def test_gemm_deterministic():
    x, w = workloads.tiny()
    a = run_w4a4(x, w, torch.float32).cpu()
    b = run_w4a4(x, w, torch.float32).cpu()
    assert torch.equal(a, b)


def run_w4a16(a_cpu, w_cpu, out_dtype, sample=None):
    M, K = a_cpu.shape
    N = w_cpu.shape[0]
    say(f"[gemm W4A16] M={M} N={N} K={K} sample={sample}")
    bp, Sb, _ = prepare_weight(w_cpu)
    ad = a_cpu.to(DEV)
    esz = 4 if out_dtype == torch.float32 else 2
    gy = Guarded(M * N * esz)
    out = gy.payload((M, N), out_dtype)
    nv.nvfp4_gemm(nv.W4A16, ad, None, None, bp, Sb, N, K, out_dtype, out=out)
    torch.cuda.synchronize()
    gy.check()
    Yg = out.float().cpu().numpy()
    A = oracle.bf16_to_f32(np_bf16(a_cpu))
    wo = np_x(w_cpu)
    SB = oracle.tensor_scale(wo)
    if sample is None:
        cols = np.arange(N)
    else:
        cols = np.unique(np.random.default_rng(N + K).integers(0, N, sample))
    bo_p, bo_s, _ = oracle.quantize(np.ascontiguousarray(wo[cols]), S=SB)
    B, _ = oracle.dequantize(bo_p, bo_s, SB)
    Y, R = oracle.gemm(A, B)
    check_gemm(Yg[:, cols], Y, R, out_dtype == torch.bfloat16, f"W4A16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (16, 96, 256), (37, 200, 1152), (300, 130, 384), (5, 48, 80),
                                   # streaming kernel (M <= 32): K split over workgroups, ragged last unit
                                   (1, 1000, 2048), (31, 1000, 2048), (7, 98, 1536), (16, 4096, 3072), (3, 200, 4096),
                                   # each activation row class of the streaming kernel (4, 8, 16, 32 rows),
                                   # full and partly filled
                                   (4, 520, 1152), (9, 300, 1152), (17, 1000, 2048), (32, 4096, 3072),
                                   # two row groups (33..64 rows)
                                   (33, 1000, 2048), (48, 130, 1152), (64, 4096, 3072),
                                   # 64 x 256 tiles: K split two / five ways, ragged M and N, 9 chunks
                                   (200, 520, 2048), (600, 520, 384), (512, 256, 4096), (1000, 300, 1152),
                                   # 128 x 256 tiles, whole-chunk stages: ragged, K split five ways
                                   (1500, 2600, 384), (2100, 300, 4096),
                                   # half-chunk stages, two workgroups per CU: ragged, K split 7 / 3 ways
                                   (3000, 2600, 384), (4100, 300, 12288), (1500, 2600, 4096)])
def test_gemm_w4a16_ragged(M, N, K):
    g = torch.Generator().manual_seed(M * 5 + N + K)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = workloads.laplace_tailed_weight(N, K, g)
    run_w4a16(a, w, torch.float32)


@pytest.mark.parametrize("M,N,K", [(1, 520, 1152), (9, 520, 1152), (17, 520, 1152), (32, 520, 1152),
                                   (50, 520, 1152), (300, 520, 1152), (1500, 2600, 384), (3000, 2600, 384)])
def test_gemm_w4a16_strided_activation(M, N, K):
    """A row-strided activation view (lda = K + 64, the padding holds 1e30 and must be ignored):
    streaming kernel for each row class, then the tiled forms: 64 x 256 tiles (M = 300), 128 x 256
    with whole-chunk stages (M = 1500) and with half-chunk stages, two workgroups per CU (M = 3000)."""
    g = torch.Generator().manual_seed(900 + M)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = workloads.laplace_tailed_weight(N, K, g)
    say(f"[gemm W4A16 strided] M={M} N={N} K={K} lda={K + 64}")
    bp, Sb, _ = prepare_weight(w)
    big = torch.full((M, K + 64), 1e30, dtype=torch.bfloat16)
    big[:, :K] = a
    ad = big.to(DEV)[:, :K]
    out = nv.nvfp4_gemm(nv.W4A16, ad, None, None, bp, Sb, N, K, torch.float32)
    torch.cuda.synchronize()
    wo = np_x(w)
    SB = oracle.tensor_scale(wo)
    bo_p, bo_s, _ = oracle.quantize(wo, S=SB)
    B, _ = oracle.dequantize(bo_p, bo_s, SB)
    Y, R = oracle.gemm(oracle.bf16_to_f32(np_bf16(a)), B)
    check_gemm(out.cpu().numpy(), Y, R, False, f"W4A16 strided {M}x{N}x{K}")


def test_gemm_w4a16_full_size():
    """The weight-only up and down projections at M = 1, 16, 256 and 4096, every output element."""
    for name, (w, acts) in workloads.w4a16().items():
        for m, a in acts.items():
            run_w4a16(a, w, torch.bfloat16)


def test_empty_tensors():
    """M == 0: dynamic quantize writes S = 0 (the oracle's maximum over no element), and
    dequantize / GEMM with an empty side return empty outputs without touching memory."""
    say("[empty] M=0 quantize / dequantize / gemm, N=0 gemm")
    K, N = 64, 96
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    S = torch.full((1,), 7.0, dtype=torch.float32, device=DEV)
    p, s, _ = nv.nvfp4_quantize(x, S, static=False)
    torch.cuda.synchronize()
    assert p.shape == (0, K // 2) and s.shape == (0, K // 16)
    assert S.item() == 0.0
    assert float(oracle.tensor_scale(np.zeros((0, K), np.uint16))) == 0.0
    y = nv.nvfp4_dequantize(p, s, S, torch.float32)
    assert y.shape == (0, K)
    g = torch.Generator().manual_seed(11)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    bp, Sb, _ = prepare_weight(w)
    out = nv.nvfp4_gemm(nv.W4A4, p, s, S, bp, Sb, N, K, torch.float32)
    out16 = nv.nvfp4_gemm(nv.W4A16, x, None, None, bp, Sb, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    assert out.shape == (0, N) and out16.shape == (0, N)
    # N == 0: an empty weight
    xa = torch.randn(5, K, generator=g).to(torch.bfloat16).to(DEV)
    pa, sa, Sa = nv.nvfp4_quantize(xa)
    we = torch.empty((0, K // 2), dtype=torch.uint8, device=DEV)
    se = torch.empty((0, K // 16), dtype=torch.uint8, device=DEV)
    bpe = nv.nvfp4_prepack_weight(we, se)
    assert bpe.numel() == 0
    oute = nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bpe, Sa, 0, K, torch.float32)
    torch.cuda.synchronize()
    assert oute.shape == (5, 0)


# ---- fake quantization (QAT) ------------------------------------------------------------------------

def oracle_fake(x_cpu, static_S, out_dtype):
    op, os_, oS = oracle.quantize(np_x(x_cpu), S=static_S)
    y32, y16 = oracle.dequantize(op, os_, oS)
    return (y32.view(np.uint32) if out_dtype == torch.float32 else y16), oS


def run_fake(x_cpu, static_S, out_dtype, ld_x=None, ld_y=None, label=""):
    M, K = x_cpu.shape
    say(f"[fake] {label} {tuple(x_cpu.shape)} {x_cpu.dtype}->{out_dtype} static={static_S} ld={ld_x},{ld_y}")
    if ld_x is not None and ld_x != K:
        big = torch.full((M, ld_x), 1e30, dtype=x_cpu.dtype)
        big[:, :K] = x_cpu
        xd = big.to(DEV)[:, :K]
    else:
        xd = x_cpu.to(DEV)
    esz = 4 if out_dtype == torch.float32 else 2
    ld_y = ld_y or K
    gy = Guarded(M * ld_y * esz)
    yb = gy.payload((M, ld_y), out_dtype)
    yb.fill_(7.0)
    y = yb[:, :K]
    Sd = (torch.tensor([static_S], dtype=torch.float32, device=DEV) if static_S is not None
          else torch.empty(1, dtype=torch.float32, device=DEV))
    nv.nvfp4_fake_quantize(xd, Sd, static=static_S is not None, out=y)
    torch.cuda.synchronize()
    gy.check()
    assert (yb[:, K:] == 7.0).all(), "padding columns of y written"
    want, oS = oracle_fake(x_cpu, static_S, out_dtype)
    assert np.float32(Sd.item()).view(np.uint32) == np.float32(oS).view(np.uint32)
    got = y.cpu().contiguous()
    got = got.view(torch.int32).numpy().view(np.uint32) if out_dtype == torch.float32 else np_bf16(got)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} outputs differ, first at {bad[0][0], bad[1][0]}"
    return y


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fake_quantize_sweep(out_dtype):
    x = workloads.sweep(4096, 1152)
    run_fake(x, None, out_dtype, label="sweep dynamic")
    xs = workloads.sweep(4096, 1152, static=True)
    run_fake(xs, workloads.SWEEP_STATIC_S, out_dtype, label="sweep static")


@pytest.mark.parametrize("M,K,ld_x,ld_y,dt,out", [
    (1, 16, 16, 16, torch.float32, torch.float32), (37, 48, 56, 64, torch.bfloat16, torch.float32),
    (255, 1168, 1168, 1176, torch.float32, torch.bfloat16), (300, 272, 280, 272, torch.bfloat16, torch.bfloat16),
])
def test_fake_quantize_ragged(M, K, ld_x, ld_y, dt, out):
    g = torch.Generator().manual_seed(M + K)
    x = (torch.randn(M, K, generator=g) * torch.exp(2 * torch.randn(M, 1, generator=g))).to(dt)
    run_fake(x, None, out, ld_x, ld_y, label="ragged dynamic")
    run_fake(x, 0.004, out, ld_x, ld_y, label="ragged static")


def test_fake_quantize_equals_quantize_then_dequantize_and_ste():
    x, _ = workloads.tiny()
    xd = x.to(DEV)
    p, s, S = nv.nvfp4_quantize(xd)
    y2 = nv.nvfp4_dequantize(p, s, S, torch.float32)
    y1, S1 = nv.nvfp4_fake_quantize(xd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)) and S1.item() == S.item()
    # straight-through estimator: the gradient passes unchanged
    xg = xd.clone().requires_grad_(True)
    yg = nv.fake_quantize_ste(xg)
    assert torch.equal(yg.detach().view(torch.int32), y1.view(torch.int32))
    gout = torch.randn_like(xg)
    yg.backward(gout)
    assert torch.equal(xg.grad, gout)
