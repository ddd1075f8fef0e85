"""Debug checks on the GPU: with nvfp4_set_debug_checks(True), a call whose device data breaks a
precondition the header states (a non-finite input or bias, a NaN scale byte, a tensor scale that
is not finite, or not > 0 where the call divides by it) raises ERR_PRECONDITION and writes nothing;
data outside the extent the call reads (row padding) is not scanned; valid calls give the same
bytes as with the checks off; calls under graph capture skip the scans.  No kernel of the product
path ever runs on the bad data: the scans stop the call first."""
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
from test_gpu_parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def debug():
    prev = nv.nvfp4_set_debug_checks(True)
    try:
        yield
    finally:
        nv.nvfp4_set_debug_checks(prev)


def rejected(label, fn, *outs):
    """fn must raise ERR_PRECONDITION and leave every output tensor as it was."""
    say(f"[debug checks] {label}: expect ERR_PRECONDITION")
    torch.cuda.synchronize()
    before = [o.clone() for o in outs]
    with pytest.raises(nv.NVFP4Error) as ei:
        fn()
    assert ei.value.status == nv.Status.ERR_PRECONDITION, str(ei.value)
    torch.cuda.synchronize()
    for o, b in zip(outs, before):
        assert torch.equal(o, b), f"{label}: an output was written"


def same_with_checks_off(label, fn):
    """fn() with the checks on returns the same tensors, bit for bit, as with them off."""
    say(f"[debug checks] {label}: valid call, checks on vs off")
    on = [t.clone() for t in fn()]
    prev = nv.nvfp4_set_debug_checks(False)
    try:
        off = [t.clone() for t in fn()]
    finally:
        nv.nvfp4_set_debug_checks(prev)
    torch.cuda.synchronize()
    for a, b in zip(on, off):
        assert torch.equal(a, b), label


def sentinel(shape, dtype=torch.uint8, val=0xA5):
    return torch.full(shape, val, dtype=dtype, device=DEV)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_quantize_rejects_non_finite_input(debug, dt, bad):
    M, K = 70, 320
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(1)).to(dt).to(DEV)
    x[41, 317] = bad  # the last block of a row
    packed, scales = sentinel((M, K // 2)), sentinel((M, K // 16))
    S = torch.full((1,), 7.0, device=DEV)
    ws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    rejected(f"dynamic quantize {dt} {bad}",
             lambda: nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=ws),
             packed, scales, S)
    S1 = torch.full((1,), 0.01, device=DEV)
    rejected(f"static quantize {dt} {bad}", lambda: nv.nvfp4_quantize(x, S1, packed=packed, scales=scales),
             packed, scales, S1)
    rejected(f"no-alloc quantize {dt} {bad}",
             lambda: nv.nvfp4_quantize_noalloc(x, S, packed, scales, static=False), packed, scales, S)
    y = sentinel((M, K), torch.float32, 3.0)
    rejected(f"fake quantize {dt} {bad}", lambda: nv.nvfp4_fake_quantize(x, out=y), y)
    mp, ms = sentinel((M, K // 2)), sentinel((M, K // 32))
    rejected(f"MX quantize {dt} {bad}", lambda: nv.nvfp4_mx_quantize(x, packed=mp, scales=ms), mp, ms)


def test_quantize_scans_only_the_logical_extent(debug):
    """A NaN in the row padding past K is not an input of the call."""
    M, K, ld = 33, 256, 288
    base = torch.randn(M, ld, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(DEV)
    base[:, K:] = float("nan")
    x = base[:, :K]
    same_with_checks_off("dynamic quantize, NaN padding", lambda: nv.nvfp4_quantize(x))
    same_with_checks_off("MX quantize, NaN padding", lambda: nv.nvfp4_mx_quantize(x))


@pytest.mark.parametrize("S_val", [0.0, -0.5, float("inf"), float("nan")])
def test_static_scale_must_be_finite_and_positive(debug, S_val):
    M, K = 16, 64
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(3)).to(DEV)
    packed, scales = sentinel((M, K // 2)), sentinel((M, K // 16))
    S = torch.tensor([S_val], dtype=torch.float32, device=DEV)
    rejected(f"static S = {S_val}", lambda: nv.nvfp4_quantize(x, S, packed=packed, scales=scales), packed, scales)
    y = sentinel((M, K), torch.float32, 3.0)
    rejected(f"static fake quantize S = {S_val}", lambda: nv.nvfp4_fake_quantize(x, S, out=y), y)


def test_dequantize_checks(debug):
    M, K = 40, 128
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(4)).to(DEV)
    p, s, S = nv.nvfp4_quantize(x)
    same_with_checks_off("dequantize", lambda: [nv.nvfp4_dequantize(p, s, S)])
    Sz = torch.zeros(1, device=DEV)  # finite: a zero tensor scale dequantizes to zeros
    same_with_checks_off("dequantize, S = 0", lambda: [nv.nvfp4_dequantize(p, s, Sz)])
    y = sentinel((M, K), torch.float32, 3.0)
    for byte in (0x7F, 0xFF):
        sb = s.clone()
        sb[M - 1, K // 16 - 1] = byte
        rejected(f"dequantize, scale byte {byte:#x}", lambda: nv.nvfp4_dequantize(p, sb, S, out=y), y)
    Sn = torch.tensor([float("nan")], device=DEV)
    rejected("dequantize, S = NaN", lambda: nv.nvfp4_dequantize(p, s, Sn, out=y), y)


def _weight(N, K, seed):
    w = (0.02 * torch.randn(N, K, generator=torch.Generator().manual_seed(seed))).to(DEV)
    wp, ws, wS = nv.nvfp4_quantize(w)
    return wp, ws, wS


def test_gemm_checks(debug):
    M, N, K = 300, 272, 384
    g = torch.Generator().manual_seed(5)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    wp, ws, wS = _weight(N, K, 6)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    a, as_, aS = nv.nvfp4_quantize(x)
    same_with_checks_off("W4A4 GEMM", lambda: [nv.nvfp4_gemm(nv.W4A4, a, as_, aS, bp, wS, N, K)])
    same_with_checks_off("W4A16 GEMM", lambda: [nv.nvfp4_gemm(nv.W4A16, x, None, None, bp, wS, N, K)])
    out = sentinel((M, N), torch.bfloat16, 3.0)

    # prepack rejects a NaN scale byte; a weight prepacked without checks is rejected by the GEMM
    wsb = ws.clone()
    wsb[N - 1, K // 16 - 1] = 0x7F
    bp_bad = sentinel((nv.nvfp4_prepacked_bytes(N, K),))
    rejected("prepack, NaN scale byte", lambda: nv.nvfp4_prepack_weight(wp, wsb, out=bp_bad), bp_bad)
    prev = nv.nvfp4_set_debug_checks(False)
    try:
        nv.nvfp4_prepack_weight(wp, wsb, out=bp_bad)
    finally:
        nv.nvfp4_set_debug_checks(prev)
    rejected("W4A4 GEMM, NaN weight scale", lambda: nv.nvfp4_gemm(nv.W4A4, a, as_, aS, bp_bad, wS, N, K, out=out), out)
    rejected("W4A16 GEMM, NaN weight scale",
             lambda: nv.nvfp4_gemm(nv.W4A16, x, None, None, bp_bad, wS, N, K, out=out), out)

    asb = as_.clone()
    asb[M - 1, 0] = 0xFF
    rejected("W4A4 GEMM, NaN activation scale", lambda: nv.nvfp4_gemm(nv.W4A4, a, asb, aS, bp, wS, N, K, out=out), out)
    Sinf = torch.tensor([float("inf")], device=DEV)
    rejected("W4A4 GEMM, S_A = inf", lambda: nv.nvfp4_gemm(nv.W4A4, a, as_, Sinf, bp, wS, N, K, out=out), out)
    rejected("W4A16 GEMM, S_B = inf", lambda: nv.nvfp4_gemm(nv.W4A16, x, None, None, bp, Sinf, N, K, out=out), out)
    xb = x.clone()
    xb[M // 2, K - 1] = float("inf")
    rejected("W4A16 GEMM, inf activation", lambda: nv.nvfp4_gemm(nv.W4A16, xb, None, None, bp, wS, N, K, out=out), out)


@pytest.mark.parametrize("M,K", [(8, 1024), (512, 4096)])
def test_gemm_checks_skinny_and_split(debug, M, K):
    """The scans stop the call before any launch path: the streaming kernel for few rows (M = 8)
    and a K split with its fp32 partials and reduction (M = 512, K = 4096)."""
    N = 512
    g = torch.Generator().manual_seed(M + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    wp, ws, wS = _weight(N, K, 15)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    a, as_, aS = nv.nvfp4_quantize(x)
    same_with_checks_off(f"W4A16 GEMM M={M} K={K}",
                         lambda: [nv.nvfp4_gemm(nv.W4A16, x, None, None, bp, wS, N, K, torch.float32)])
    same_with_checks_off(f"W4A4 GEMM M={M} K={K}",
                         lambda: [nv.nvfp4_gemm(nv.W4A4, a, as_, aS, bp, wS, N, K, torch.float32)])
    out = sentinel((M, N), torch.float32, 3.0)
    xb = x.clone()
    xb[M - 1, 0] = float("nan")
    rejected(f"W4A16 GEMM M={M} K={K}, NaN activation",
             lambda: nv.nvfp4_gemm(nv.W4A16, xb, None, None, bp, wS, N, K, out=out), out)
    asb = as_.clone()
    asb[0, K // 16 - 1] = 0x7F
    rejected(f"W4A4 GEMM M={M} K={K}, NaN activation scale",
             lambda: nv.nvfp4_gemm(nv.W4A4, a, asb, aS, bp, wS, N, K, out=out), out)


def test_gemm_strided_activation_padding_not_scanned(debug):
    """W4A4 with lda > K: NaN scale bytes in the padding columns of the activation scales are not
    read by the call and do not trip the checks; one in the last column read does."""
    M, N, K, lda = 130, 160, 256, 384
    xw = torch.randn(M, lda, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16).to(DEV)
    pw, sw, S = nv.nvfp4_quantize(xw)
    sw[:, K // 16:] = 0xFF
    a, as_ = pw[:, :K // 2], sw[:, :K // 16]
    wp, ws, wS = _weight(N, K, 9)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    same_with_checks_off("W4A4 GEMM, NaN scale padding",
                         lambda: [nv.nvfp4_gemm(nv.W4A4, a, as_, S, bp, wS, N, K, torch.float32)])
    sw[M - 1, K // 16 - 1] = 0xFF
    out = sentinel((M, N), torch.float32, 3.0)
    rejected("W4A4 GEMM, NaN scale in the last column read",
             lambda: nv.nvfp4_gemm(nv.W4A4, a, as_, S, bp, wS, N, K, out=out), out)


def test_requant_checks(debug):
    M, N, K = 256, 512, 256
    g = torch.Generator().manual_seed(10)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    bias = (0.5 * torch.randn(N, generator=g)).to(DEV)
    wp, ws, wS = _weight(N, K, 11)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    a, as_, aS = nv.nvfp4_quantize(x)
    So = torch.tensor([0.002], device=DEV)
    same_with_checks_off("requantizing GEMM", lambda: nv.nvfp4_gemm_requant(
        nv.W4A4, a, as_, aS, bp, wS, N, K, So, bias=bias, act=nv.ACT_GELU_TANH))
    packed, scales = sentinel((M, N // 2)), sentinel((M, N // 16))
    bb = bias.clone()
    bb[N - 1] = float("nan")
    rejected("requantizing GEMM, NaN bias", lambda: nv.nvfp4_gemm_requant(
        nv.W4A4, a, as_, aS, bp, wS, N, K, So, bias=bb, packed=packed, scales=scales), packed, scales)
    for v in (0.0, float("inf")):
        Sb = torch.tensor([v], device=DEV)
        rejected(f"requantizing GEMM, output S = {v}", lambda: nv.nvfp4_gemm_requant(
            nv.W4A16, x, None, None, bp, wS, N, K, Sb, packed=packed, scales=scales), packed, scales)


def test_mx_checks(debug):
    M, N, K = 96, 128, 256
    g = torch.Generator().manual_seed(12)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).to(DEV)
    a, as_ = nv.nvfp4_mx_quantize(x)
    b, bs = nv.nvfp4_mx_quantize(w)
    same_with_checks_off("MX GEMM", lambda: [nv.nvfp4_mx_gemm(a, as_, b, bs)])
    same_with_checks_off("MX dequantize", lambda: [nv.nvfp4_mx_dequantize(a, as_)])
    bsb = bs.clone()
    bsb[N - 1, K // 32 - 1] = 0xFF
    out = sentinel((M, N), torch.bfloat16, 3.0)
    rejected("MX GEMM, 0xFF weight scale", lambda: nv.nvfp4_mx_gemm(a, as_, b, bsb, out=out), out)
    y = sentinel((N, K), torch.float32, 3.0)
    rejected("MX dequantize, 0xFF scale", lambda: nv.nvfp4_mx_dequantize(b, bsb, out=y), y)


def test_captured_calls_skip_the_scans(debug):
    """Under graph capture the scans cannot wait on the stream, so they are skipped: the captured
    quantize + GEMM replays equal the eager result."""
    M, N, K = 128, 256, 512
    g = torch.Generator().manual_seed(13)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    wp, ws, wS = _weight(N, K, 14)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    S = torch.empty(1, dtype=torch.float32, device=DEV)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)

    def run():
        nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws)
        nv.nvfp4_gemm(nv.W4A4, packed, scales, S, bp, wS, N, K, torch.float32, out=y)

    say("[debug checks] graph capture with the checks on")
    run()
    torch.cuda.synchronize()
    ref = (packed.clone(), scales.clone(), S.clone(), y.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gr, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (packed, scales, S, y):
            t.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for got, exp in zip((packed, scales, S, y), ref):
            assert torch.equal(got, exp), f"replay {rep} differs"
