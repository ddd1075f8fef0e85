"""C-ABI contract tests that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments on the host before any HIP call (fake device pointers are
never dereferenced because validation fails first)."""
import ctypes
import os
import re

import pytest

import nvfp4_quantized_gemm_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

P = ctypes.c_void_p(0x10000)     # 16-byte aligned fake device pointer (never dereferenced)
P8 = ctypes.c_void_p(0x10008)    # 8-byte aligned only
PODD = ctypes.c_void_p(0x10001)  # misaligned
NULL = None


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return nv.lib()


def test_exports_every_header_symbol(L):
    funcs = header_functions()
    assert len(funcs) >= 10
    for f in funcs:
        assert hasattr(L, f), f
    assert sorted(funcs) == sorted(nv.EXPORTED)


def test_version_and_status_strings(L):
    assert L.nvfp4_abi_version() == 3
    for s in nv.Status:
        assert len(L.nvfp4_status_string(int(s))) > 0
    assert L.nvfp4_status_string(99) == b"unknown status"
    assert b"precondition" in L.nvfp4_status_string(int(nv.Status.ERR_PRECONDITION))


def test_debug_checks_toggle_and_validation_order(L):
    """The switch returns the previous setting; with the checks on, host-side validation still
    comes first (the scans need a device and run only after the device check)."""
    prev = L.nvfp4_set_debug_checks(1)
    try:
        assert L.nvfp4_set_debug_checks(1) == 1
        assert q(L, K=24) == nv.Status.ERR_SHAPE
        assert q(L, x=PODD) == nv.Status.ERR_ALIGN
        assert q(L, ws=NULL) == nv.Status.ERR_WORKSPACE
        assert q(L) in (nv.Status.ERR_HIP, nv.Status.ERR_DEVICE)  # no GPU here: stops at the device check
        assert L.nvfp4_set_debug_checks(0) == 1
        assert L.nvfp4_set_debug_checks(0) == 0
    finally:
        L.nvfp4_set_debug_checks(prev)


@pytest.mark.parametrize("env,expect", [(None, 0), ("0", 0), ("", 0), ("1", 1), ("yes", 1)])
def test_debug_checks_initial_setting_from_environment(env, expect):
    """NVFP4_DEBUG set and not "0" turns the checks on in a fresh process (read on first use)."""
    import subprocess
    import sys
    code = ("import ctypes; L = ctypes.CDLL(%r); L.nvfp4_set_debug_checks.argtypes = [ctypes.c_int]; "
            "print(L.nvfp4_set_debug_checks(0))" % nv.LIB_PATH)
    e = {k: v for k, v in os.environ.items() if k != "NVFP4_DEBUG"}
    if env is not None:
        e["NVFP4_DEBUG"] = env
    r = subprocess.run([sys.executable, "-c", code], env=e, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == str(expect)


def test_size_queries(L):
    assert L.nvfp4_prepacked_bytes(1152, 1152) == 36 * 9 * 2304
    assert L.nvfp4_prepacked_bytes(33, 16) == 2 * 1 * 2304
    assert L.nvfp4_prepacked_bytes(0, 128) == 0
    assert L.nvfp4_prepacked_bytes(32, 24) == 0
    assert L.nvfp4_quantize_workspace_bytes(4096, 1152) >= 4
    assert L.nvfp4_gemm_workspace_bytes(0, 4096, 1152, 1152) >= 0
    assert L.nvfp4_gemm_workspace_bytes(7, 4096, 1152, 1152) == 0


def q(L, x=P, dt=nv.BF16, M=4, K=32, ld=32, packed=P, scales=P, S=P, mode=nv.SCALE_DYNAMIC, ws=P, wsb=4096):
    return L.nvfp4_quantize(x, dt, M, K, ld, packed, scales, S, mode, ws, wsb, None)


def test_quantize_validation(L):
    S = nv.Status
    assert q(L, x=NULL) == S.ERR_NULL
    assert q(L, packed=NULL) == S.ERR_NULL
    assert q(L, S=NULL) == S.ERR_NULL
    assert q(L, dt=7) == S.ERR_DTYPE
    assert q(L, mode=5) == S.ERR_MODE
    assert q(L, M=-1) == S.ERR_SHAPE
    assert q(L, K=24, ld=24) == S.ERR_SHAPE
    assert q(L, K=0, ld=0) == S.ERR_SHAPE
    assert q(L, ld=16) == S.ERR_STRIDE
    assert q(L, x=PODD) == S.ERR_ALIGN
    assert q(L, ld=36) == S.ERR_ALIGN            # 72-byte bf16 row pitch
    assert q(L, packed=ctypes.c_void_p(0x10004)) == S.ERR_ALIGN
    assert q(L, ws=NULL) == S.ERR_WORKSPACE
    assert q(L, wsb=4) == S.ERR_WORKSPACE


def test_dequantize_validation(L):
    S = nv.Status
    d = lambda **kw: L.nvfp4_dequantize(kw.get("p", P), kw.get("s", P), kw.get("ts", P), kw.get("M", 4),
                                        kw.get("K", 32), kw.get("y", P), kw.get("dt", nv.F32), kw.get("ld", 32), None)
    assert d(p=NULL) == S.ERR_NULL
    assert d(y=NULL) == S.ERR_NULL
    assert d(dt=3) == S.ERR_DTYPE
    assert d(K=17) == S.ERR_SHAPE
    assert d(ld=8) == S.ERR_STRIDE
    assert d(y=PODD) == S.ERR_ALIGN
    assert d(ld=33) == S.ERR_ALIGN


def test_fake_quantize_validation(L):
    S = nv.Status
    f = lambda **kw: L.nvfp4_fake_quantize(kw.get("x", P), kw.get("dt", nv.BF16), kw.get("M", 4), kw.get("K", 32),
                                           kw.get("ld", 32), kw.get("y", P), kw.get("ydt", nv.F32),
                                           kw.get("ldy", 32), kw.get("S", P), kw.get("mode", nv.SCALE_DYNAMIC),
                                           kw.get("ws", P), kw.get("wsb", 4096), None)
    assert f(S=NULL) == S.ERR_NULL
    assert f(y=NULL) == S.ERR_NULL
    assert f(ydt=9) == S.ERR_DTYPE
    assert f(mode=3) == S.ERR_MODE
    assert f(K=40, ld=40, ldy=40) == S.ERR_SHAPE
    assert f(ldy=16) == S.ERR_STRIDE
    assert f(y=P8) == S.ERR_ALIGN
    assert f(ydt=nv.BF16, ldy=36) == S.ERR_ALIGN
    assert f(ws=NULL) == S.ERR_WORKSPACE
    assert f(x=NULL, y=NULL, M=0, mode=nv.SCALE_STATIC, ws=NULL, wsb=0) == S.OK


def test_prepack_validation(L):
    S = nv.Status
    assert L.nvfp4_prepack_weight(NULL, P, 32, 128, P, None) == S.ERR_NULL
    assert L.nvfp4_prepack_weight(P, P, 32, 120, P, None) == S.ERR_SHAPE
    assert L.nvfp4_prepack_weight(P, P, 32, 128, P8, None) == S.ERR_ALIGN
    assert L.nvfp4_unpack_weight(P, -1, 128, P, P, None) == S.ERR_SHAPE


def g(L, mode=nv.W4A4, a=P, asc=P, ats=P, b=P, bts=P, M=64, N=64, K=128, lda=128, c=P, dt=nv.BF16, ldc=64,
      ws=NULL, wsb=0):
    return L.nvfp4_gemm(mode, a, asc, ats, b, bts, M, N, K, lda, c, dt, ldc, ws, wsb, None)


def test_gemm_validation(L):
    S = nv.Status
    assert g(L, mode=9) == S.ERR_MODE
    assert g(L, a=NULL) == S.ERR_NULL
    assert g(L, asc=NULL) == S.ERR_NULL
    assert g(L, mode=nv.W4A16) == S.ERR_NULL    # W4A16 must not pass A scales
    assert g(L, dt=4) == S.ERR_DTYPE
    assert g(L, N=-1) == S.ERR_SHAPE
    assert g(L, M=-1) == S.ERR_SHAPE
    assert g(L, K=100, lda=112) == S.ERR_SHAPE
    assert g(L, lda=64) == S.ERR_STRIDE
    assert g(L, ldc=32) == S.ERR_STRIDE
    assert g(L, lda=136) == S.ERR_STRIDE       # W4A4 row pitch must hold whole scale blocks
    assert g(L, b=P8) == S.ERR_ALIGN
    assert g(L, c=PODD) == S.ERR_ALIGN
    assert g(L, mode=nv.W4A16, asc=NULL, ats=NULL, a=P8) == S.ERR_ALIGN


def rq(L, mode=nv.W4A4, a=P, asc=P, ats=P, b=P, bts=P, M=64, N=64, K=128, lda=128, bias=NULL, act=0, ots=P,
       op=P, osc=P, y=NULL, ldy=0, ws=NULL, wsb=0):
    return L.nvfp4_gemm_requant(mode, a, asc, ats, b, bts, M, N, K, lda, bias, act, ots, op, osc, y, ldy, ws, wsb,
                                None)


def test_gemm_requant_validation(L):
    S = nv.Status
    assert rq(L, mode=9) == S.ERR_MODE
    assert rq(L, act=7) == S.ERR_MODE
    assert rq(L, N=40) == S.ERR_SHAPE              # output blocks run along N: N % 16 == 0
    assert rq(L, N=-16) == S.ERR_SHAPE
    assert rq(L, K=100, lda=112) == S.ERR_SHAPE
    assert rq(L, ots=NULL) == S.ERR_NULL
    assert rq(L, op=NULL) == S.ERR_NULL
    assert rq(L, osc=NULL) == S.ERR_NULL
    assert rq(L, mode=nv.W4A16) == S.ERR_NULL      # W4A16 must not pass A scales
    assert rq(L, lda=64) == S.ERR_STRIDE
    assert rq(L, y=P, ldy=32) == S.ERR_STRIDE       # ld_y >= N
    assert rq(L, y=P, ldy=66) == S.ERR_STRIDE       # ld_y % 4 == 0
    assert rq(L, bias=P8) == S.ERR_ALIGN
    assert rq(L, op=P8) == S.ERR_ALIGN
    assert rq(L, y=P8, ldy=64) == S.ERR_ALIGN
    # a split-K shape needs the fp32 partials; so does the generic kernel (K % 128 != 0)
    need = L.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, 512, 512, 4096)
    assert need >= 4 * 512 * 512 * 2
    assert rq(L, M=512, N=512, K=4096, lda=4096) == S.ERR_WORKSPACE
    assert rq(L, M=512, N=512, K=4096, lda=4096, ws=P, wsb=need - 1) == S.ERR_WORKSPACE
    assert L.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, 64, 96, 48) == 64 * 96 * 4
    assert L.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, 64, 40, 128) == 0   # invalid N
    # empty outputs touch nothing
    assert rq(L, a=NULL, asc=NULL, ats=NULL, b=NULL, bts=NULL, ots=NULL, op=NULL, osc=NULL, M=0) == S.OK
    assert rq(L, a=NULL, asc=NULL, ats=NULL, b=NULL, bts=NULL, ots=NULL, op=NULL, osc=NULL, N=0) == S.OK


def test_workspace_queries_follow_the_activation_pitch(L):
    """The workspace a GEMM call needs is that of the plan its own lda selects: a W4A4 row pitch that
    is not a multiple of 128 codes runs the generic kernel, whose NVFP4-output form stages fp32
    values in the workspace.  The entry points check the caller's buffer against that plan and
    return ERR_WORKSPACE before any device work when it is short (NVFP4-DiT page, Methodology
    section 3: the packed operands of the next W4A4 product)."""
    S = nv.Status
    M, N, K = 300, 272, 384
    # lda = K and K + 128: 128 x 128 tiles, no partials; K + 16: the generic kernel
    assert L.nvfp4_gemm_requant_workspace_bytes_ld(nv.W4A4, M, N, K, K) == 0
    assert L.nvfp4_gemm_requant_workspace_bytes_ld(nv.W4A4, M, N, K, K + 128) == 0
    assert L.nvfp4_gemm_requant_workspace_bytes_ld(nv.W4A4, M, N, K, K + 16) == M * N * 4
    assert L.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, M, N, K) == 0
    # the call with a pitch of 400 codes and no workspace is refused on the host
    assert rq(L, M=M, N=N, K=K, lda=400) == S.ERR_WORKSPACE
    assert rq(L, M=M, N=N, K=K, lda=400, ws=P, wsb=M * N * 4 - 1) == S.ERR_WORKSPACE
    # the bf16 / fp32 output of the generic kernel needs none
    assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A4, M, N, K, K + 16) == 0
    # a split-K plan (16 tiles, 32 chunks: several fp32 partials) with lda = K or K + 128, none for
    # the generic kernel
    M, N, K = 512, 512, 4096
    need = L.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K)
    assert need >= 2 * M * N * 4 and need % (M * N * 4) == 0
    for ld in (K, K + 128):
        assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A4, M, N, K, ld) == need
        assert L.nvfp4_gemm_requant_workspace_bytes_ld(nv.W4A4, M, N, K, ld) == need
    assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A4, M, N, K, K + 16) == 0
    assert L.nvfp4_gemm_requant_workspace_bytes_ld(nv.W4A4, M, N, K, K + 16) == M * N * 4
    assert g(L, M=M, N=N, K=K, lda=K + 128, ldc=N, ws=P, wsb=need - 16) == S.ERR_WORKSPACE
    # W4A16 rows <= 64 stream unless 32 rows of the pitch pass 2 GiB; the tiled plan then decides
    lda = 1 << 26
    assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A16, 16, 3072, 12288, 12288) == \
        L.nvfp4_gemm_workspace_bytes(nv.W4A16, 16, 3072, 12288)
    need_tiled = L.nvfp4_gemm_workspace_bytes_ld(nv.W4A16, 16, 3072, 12288, lda)
    assert need_tiled in (0,) or need_tiled % (16 * 3072 * 4) == 0
    # a pitch below K is not a call: the queries return 0
    assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A4, 64, 64, 128, 112) == 0


def test_gemm_extent_bounds(L):
    """K and the activation pitch are bounded like M and N (the kernels take 32-bit depths)."""
    S = nv.Status
    big = 1 << 30
    assert g(L, M=1, N=16, K=big, lda=big, ldc=16) == S.ERR_SHAPE
    assert rq(L, M=1, N=16, K=big, lda=big) == S.ERR_SHAPE
    assert g(L, M=1 << 20, N=64, K=128, lda=1 << 21, ldc=64) == S.ERR_SHAPE   # M * lda > 2^40
    assert L.nvfp4_gemm_workspace_bytes_ld(nv.W4A4, 1, 16, big, big) == 0


def test_empty_tensors_touch_nothing(L):
    """M == 0 (or N == 0 for the GEMM and the weight calls) is valid: the call returns OK at once,
    before any device work, with NULL pointers for the empty arrays.  (Dynamic quantization of an
    empty tensor still writes S = 0 on the device; the GPU tests cover it.)"""
    S = nv.Status
    assert q(L, x=NULL, M=0, packed=NULL, scales=NULL, mode=nv.SCALE_STATIC, ws=NULL, wsb=0) == S.OK
    assert q(L, x=NULL, M=0, packed=NULL, scales=NULL, S=NULL) == S.ERR_NULL   # S is still needed
    assert q(L, x=NULL, M=0, K=24, ld=24, mode=nv.SCALE_STATIC) == S.ERR_SHAPE
    assert L.nvfp4_dequantize(NULL, NULL, NULL, 0, 32, NULL, nv.BF16, 32, None) == S.OK
    assert L.nvfp4_dequantize(NULL, NULL, NULL, 0, 30, NULL, nv.BF16, 32, None) == S.ERR_SHAPE
    assert L.nvfp4_prepack_weight(NULL, NULL, 0, 128, NULL, None) == S.OK
    assert L.nvfp4_unpack_weight(NULL, 0, 128, NULL, NULL, None) == S.OK
    assert g(L, a=NULL, asc=NULL, ats=NULL, b=NULL, bts=NULL, c=NULL, M=0) == S.OK
    assert g(L, a=NULL, asc=NULL, ats=NULL, b=NULL, bts=NULL, c=NULL, N=0, ldc=0) == S.OK
    assert g(L, mode=nv.W4A16, a=NULL, asc=NULL, ats=NULL, b=NULL, bts=NULL, c=NULL, M=0) == S.OK
    assert L.nvfp4_gemm_workspace_bytes(0, 0, 64, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(nv, "_lib", None)
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libnvfp4.so not found"):
        nv.lib()
