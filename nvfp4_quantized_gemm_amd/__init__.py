"""Python binding of libnvfp4 (NVFP4 quantize / dequantize / prepack / GEMM for MI355X, gfx950).

Thin ctypes layer over the C ABI in ``include/nvfp4.h``: it allocates outputs and workspaces with
PyTorch (device memory and streams only), passes raw device pointers and the current HIP stream,
and turns a non-zero status into an exception.  Every step of the computation runs in the HIP
kernels of ``libnvfp4.so``; there is no fallback.  The function names mirror the C entry points.
"""
from __future__ import annotations

import ctypes
import os
from enum import IntEnum

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")


class Status(IntEnum):
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_STRIDE = 3
    ERR_ALIGN = 4
    ERR_DTYPE = 5
    ERR_MODE = 6
    ERR_WORKSPACE = 7
    ERR_HIP = 8
    ERR_DEVICE = 9
    ERR_PRECONDITION = 10


F32, BF16 = 0, 1
W4A4, W4A16 = 0, 1
SCALE_DYNAMIC, SCALE_STATIC = 0, 1

EXPORTED = (
    "nvfp4_status_string", "nvfp4_abi_version",
    "nvfp4_quantize_workspace_bytes", "nvfp4_quantize",
    "nvfp4_dequantize", "nvfp4_fake_quantize",
    "nvfp4_prepacked_bytes", "nvfp4_prepack_weight", "nvfp4_unpack_weight",
    "nvfp4_gemm_workspace_bytes", "nvfp4_gemm_workspace_bytes_ld", "nvfp4_gemm",
    "nvfp4_gemm_requant_workspace_bytes", "nvfp4_gemm_requant_workspace_bytes_ld", "nvfp4_gemm_requant",
    "nvfp4_quantize_bs", "nvfp4_dequantize_bs", "nvfp4_fake_quantize_bs", "nvfp4_prepack_weight_bs",
    "nvfp4_unpack_weight_bs", "nvfp4_gemm_bs", "nvfp4_gemm_requant_bs",
    "nvfp4_mx_quantize", "nvfp4_mx_dequantize", "nvfp4_mx_gemm",
    "nvfp4_quantize_noalloc", "nvfp4_set_debug_checks",
)

_lib = None
_vp, _i64, _sz, _i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = Status(status)
        super().__init__(f"{call}: {self.status.name} ({lib().nvfp4_status_string(status).decode()})")


def lib():
    """The loaded libnvfp4 (ctypes.CDLL).  Raises if the HIP library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libnvfp4.so not found at {LIB_PATH}; build it with "
                           "`python nvfp4_quantized_gemm_amd/build.py` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [_i]
    L.nvfp4_abi_version.restype = _i
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_set_debug_checks.restype = _i
    L.nvfp4_set_debug_checks.argtypes = [_i]
    L.nvfp4_quantize_workspace_bytes.restype = _sz
    L.nvfp4_quantize_workspace_bytes.argtypes = [_i64, _i64]
    L.nvfp4_quantize.restype = _i
    L.nvfp4_quantize.argtypes = [_vp, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i, _vp, _sz, _vp]
    L.nvfp4_fake_quantize.restype = _i
    L.nvfp4_fake_quantize.argtypes = [_vp, _i, _i64, _i64, _i64, _vp, _i, _i64, _vp, _i, _vp, _sz, _vp]
    L.nvfp4_dequantize.restype = _i
    L.nvfp4_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _i, _i64, _vp]
    L.nvfp4_prepacked_bytes.restype = _sz
    L.nvfp4_prepacked_bytes.argtypes = [_i64, _i64]
    L.nvfp4_prepack_weight.restype = _i
    L.nvfp4_prepack_weight.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
    L.nvfp4_unpack_weight.restype = _i
    L.nvfp4_unpack_weight.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    L.nvfp4_gemm_workspace_bytes.restype = _sz
    L.nvfp4_gemm_workspace_bytes.argtypes = [_i, _i64, _i64, _i64]
    L.nvfp4_gemm_workspace_bytes_ld.restype = _sz
    L.nvfp4_gemm_workspace_bytes_ld.argtypes = [_i, _i64, _i64, _i64, _i64]
    L.nvfp4_gemm.restype = _i
    L.nvfp4_gemm.argtypes = [_i, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i, _i64, _vp, _sz, _vp]
    L.nvfp4_gemm_requant_workspace_bytes.restype = _sz
    L.nvfp4_gemm_requant_workspace_bytes.argtypes = [_i, _i64, _i64, _i64]
    L.nvfp4_gemm_requant_workspace_bytes_ld.restype = _sz
    L.nvfp4_gemm_requant_workspace_bytes_ld.argtypes = [_i, _i64, _i64, _i64, _i64]
    L.nvfp4_gemm_requant.restype = _i
    L.nvfp4_gemm_requant.argtypes = [_i, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i, _vp, _vp, _vp,
                                     _vp, _i64, _vp, _sz, _vp]
    L.nvfp4_quantize_bs.restype = _i
    L.nvfp4_quantize_bs.argtypes = [_vp, _i, _i64, _i64, _i64, _i, _vp, _vp, _vp, _i, _vp, _sz, _vp]
    L.nvfp4_fake_quantize_bs.restype = _i
    L.nvfp4_fake_quantize_bs.argtypes = [_vp, _i, _i64, _i64, _i64, _i, _vp, _i, _i64, _vp, _i, _vp, _sz, _vp]
    L.nvfp4_dequantize_bs.restype = _i
    L.nvfp4_dequantize_bs.argtypes = [_vp, _vp, _vp, _i64, _i64, _i, _vp, _i, _i64, _vp]
    L.nvfp4_prepack_weight_bs.restype = _i
    L.nvfp4_prepack_weight_bs.argtypes = [_vp, _vp, _i64, _i64, _i, _vp, _vp]
    L.nvfp4_unpack_weight_bs.restype = _i
    L.nvfp4_unpack_weight_bs.argtypes = [_vp, _i64, _i64, _i, _vp, _vp, _vp]
    L.nvfp4_gemm_bs.restype = _i
    L.nvfp4_gemm_bs.argtypes = [_i, _vp, _vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i, _i64, _vp, _sz, _vp]
    L.nvfp4_gemm_requant_bs.restype = _i
    L.nvfp4_gemm_requant_bs.argtypes = [_i, _vp, _vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i, _vp, _vp,
                                        _vp, _vp, _i64, _vp, _sz, _vp]
    L.nvfp4_mx_quantize.restype = _i
    L.nvfp4_mx_quantize.argtypes = [_vp, _i, _i64, _i64, _i64, _vp, _vp, _vp]
    L.nvfp4_mx_dequantize.restype = _i
    L.nvfp4_mx_dequantize.argtypes = [_vp, _vp, _i64, _i64, _vp, _i, _i64, _vp]
    L.nvfp4_mx_gemm.restype = _i
    L.nvfp4_quantize_noalloc.restype = _i
    L.nvfp4_quantize_noalloc.argtypes = [_vp, _i, _i64, _i64, _i64, _i, _vp, _vp, _vp, _i, _vp]
    L.nvfp4_mx_gemm.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i, _i64, _vp]
    _lib = L
    return L


def _check(status: int, call: str):
    if status != 0:
        raise NVFP4Error(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt}; libnvfp4 takes float32 or bfloat16")


def nvfp4_set_debug_checks(enable: bool) -> bool:
    """Turn the library's device-data precondition scans on or off for every later call; returns
    the previous setting.  When on, a call whose inputs hold a non-finite value, a NaN scale byte
    or an invalid tensor scale raises NVFP4Error(ERR_PRECONDITION) and launches nothing; every call
    then waits on its stream.  The initial setting comes from the NVFP4_DEBUG environment variable."""
    return bool(lib().nvfp4_set_debug_checks(1 if enable else 0))


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along K")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.shape[0], t.shape[1], t.stride(0)


# ---- quantize / dequantize ----------------------------------------------------------------------

def nvfp4_quantize_workspace_bytes(M: int, K: int) -> int:
    return int(lib().nvfp4_quantize_workspace_bytes(M, K))


def nvfp4_quantize(x: torch.Tensor, tensor_scale: torch.Tensor | None = None, *, static: bool | None = None,
                   packed=None, scales=None, workspace=None, block_size: int = 16, stream=None):
    """Quantize x [M, K] (fp32 or bf16, device).

    static=False (the default when tensor_scale is None): dynamic scale, computed on the device and
    written to tensor_scale (allocated when None).  static=True (the default when tensor_scale is
    given): tensor_scale holds the caller's S.  block_size: values per scale byte (16, 32 or 64).
    Returns (packed u8 [M, K/2], scales u8 [M, K/block_size], S f32 [1])."""
    M, K, ld = _rows(x, "x")
    dev = x.device
    if packed is None:
        packed = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, max(K // block_size, 0)), dtype=torch.uint8, device=dev)
    if static is None:
        static = tensor_scale is not None
    dynamic = not static
    if tensor_scale is None:
        if static:
            raise ValueError("static quantization needs tensor_scale")
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    S = tensor_scale
    ws_bytes = 0
    if dynamic:
        ws_bytes = nvfp4_quantize_workspace_bytes(M, K)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().nvfp4_quantize_bs(_ptr(x), _dtype_code(x.dtype), M, K, ld, block_size, _ptr(packed), _ptr(scales),
                                 _ptr(S), SCALE_DYNAMIC if dynamic else SCALE_STATIC, _ptr(workspace), ws_bytes,
                                 _stream(stream))
    _check(st, "nvfp4_quantize_bs")
    return packed, scales, S


def nvfp4_quantize_noalloc(x: torch.Tensor, tensor_scale: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                           *, static: bool = False, block_size: int = 16, stream=None):
    """nvfp4_quantize into caller-given outputs with no workspace: the dynamic pass uses the library's
    own device scratch, so neither this call nor the library allocates anything.  tensor_scale is
    written (dynamic) or read (static).  Calls that overlap on one GPU race (they share the scratch)."""
    M, K, ld = _rows(x, "x")
    st = lib().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x.dtype), M, K, ld, block_size, _ptr(packed),
                                      _ptr(scales), _ptr(tensor_scale), SCALE_STATIC if static else SCALE_DYNAMIC,
                                      _stream(stream))
    _check(st, "nvfp4_quantize_noalloc")
    return packed, scales, tensor_scale


def _block_of(K: int, scales: torch.Tensor) -> int:
    """Block size of a canonical scale tensor [rows, K / block_size]."""
    n = scales.shape[1] if scales.dim() == 2 else 0
    return K // n if n else 16


def nvfp4_dequantize(packed: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor,
                     dtype: torch.dtype = torch.float32, *, out=None, stream=None) -> torch.Tensor:
    """y = dequantize(packed, scales, S); the block size is read from the shape of scales."""
    M, K = packed.shape[0], packed.shape[1] * 2
    if out is None:
        out = torch.empty((M, K), dtype=dtype, device=packed.device)
    _, _, ld = _rows(out, "out")
    st = lib().nvfp4_dequantize_bs(_ptr(packed), _ptr(scales), _ptr(tensor_scale), M, K, _block_of(K, scales),
                                   _ptr(out), _dtype_code(out.dtype), ld, _stream(stream))
    _check(st, "nvfp4_dequantize_bs")
    return out


def nvfp4_fake_quantize(x: torch.Tensor, tensor_scale: torch.Tensor | None = None, *, static: bool | None = None,
                        out_dtype: torch.dtype | None = None, out=None, workspace=None, block_size: int = 16,
                        stream=None):
    """y = dequantize(quantize(x)) in one pass (x [M, K] fp32 or bf16 on the device).  Scale
    arguments as for nvfp4_quantize.  Returns (y, S)."""
    M, K, ld = _rows(x, "x")
    dev = x.device
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype or x.dtype, device=dev)
    _, _, ld_y = _rows(out, "out")
    if static is None:
        static = tensor_scale is not None
    if tensor_scale is None:
        if static:
            raise ValueError("static quantization needs tensor_scale")
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = 0
    if not static:
        ws_bytes = nvfp4_quantize_workspace_bytes(M, K)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().nvfp4_fake_quantize_bs(_ptr(x), _dtype_code(x.dtype), M, K, ld, block_size, _ptr(out),
                                      _dtype_code(out.dtype), ld_y, _ptr(tensor_scale),
                                      SCALE_STATIC if static else SCALE_DYNAMIC, _ptr(workspace), ws_bytes,
                                      _stream(stream))
    _check(st, "nvfp4_fake_quantize_bs")
    return out, tensor_scale


class FakeQuantizeSTE(torch.autograd.Function):
    """Quantization-aware-training op: forward is NVFP4 fake quantization (nvfp4_fake_quantize, output
    in x's dtype), backward is the straight-through estimator, i.e. the incoming gradient unchanged."""

    @staticmethod
    def forward(ctx, x, tensor_scale=None, block_size=16):
        y, _ = nvfp4_fake_quantize(x.contiguous(), tensor_scale, block_size=block_size)
        return y

    @staticmethod
    def backward(ctx, grad_out):
        return grad_out, None, None


def fake_quantize_ste(x: torch.Tensor, tensor_scale: torch.Tensor | None = None, block_size: int = 16) -> torch.Tensor:
    """NVFP4 fake quantization with a straight-through gradient (dynamic scale when tensor_scale is
    None, else the given static scale; block_size values per scale byte: 16, 32 or 64)."""
    return FakeQuantizeSTE.apply(x, tensor_scale, block_size)


# ---- weight prepack -------------------------------------------------------------------------------

def nvfp4_prepacked_bytes(N: int, K: int) -> int:
    return int(lib().nvfp4_prepacked_bytes(N, K))


def nvfp4_prepack_weight(packed: torch.Tensor, scales: torch.Tensor, *, out=None, stream=None) -> torch.Tensor:
    N, K = packed.shape[0], packed.shape[1] * 2
    nbytes = nvfp4_prepacked_bytes(N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    st = lib().nvfp4_prepack_weight_bs(_ptr(packed), _ptr(scales), N, K, _block_of(K, scales), _ptr(out),
                                       _stream(stream))
    _check(st, "nvfp4_prepack_weight_bs")
    return out


def nvfp4_unpack_weight(prepacked: torch.Tensor, N: int, K: int, *, block_size: int = 16, stream=None):
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=prepacked.device)
    scales = torch.empty((N, K // block_size), dtype=torch.uint8, device=prepacked.device)
    st = lib().nvfp4_unpack_weight_bs(_ptr(prepacked), N, K, block_size, _ptr(packed), _ptr(scales),
                                      _stream(stream))
    _check(st, "nvfp4_unpack_weight_bs")
    return packed, scales


# ---- GEMM -------------------------------------------------------------------------------------------

def nvfp4_gemm_workspace_bytes(mode: int, M: int, N: int, K: int, lda: int | None = None) -> int:
    """Workspace bytes of nvfp4_gemm for an activation with row pitch lda (elements; K when None)."""
    return int(lib().nvfp4_gemm_workspace_bytes_ld(mode, M, N, K, K if lda is None else lda))


def _activation_pitch(mode: int, a: torch.Tensor, a_scales, a_block_size):
    """(lda in elements, W4A4 activation block size) of a GEMM's A operand.  W4A4: a is packed codes
    [M, K/2] (a row-strided view is allowed: lda = 2 * its row stride) and a_scales the matching
    [M, K/block] view of [M, lda/block] bytes; the block size is a_block_size, else lda over the scale
    tensor's row stride.  W4A16: a is bf16 [M, K] with unit stride along K."""
    if mode != W4A4:
        _, _, lda = _rows(a, "a")
        return lda, 16
    lda = a.stride(0) * 2
    if a_block_size is not None:
        return lda, int(a_block_size)
    if a_scales is not None and a_scales.dim() == 2 and a_scales.shape[0] >= 1 and a_scales.stride(0) > 0:
        return lda, lda // a_scales.stride(0)
    return lda, _block_of(lda, a_scales)


def nvfp4_gemm(mode: int, a: torch.Tensor, a_scales, a_tensor_scale, b_prepacked: torch.Tensor,
               b_tensor_scale: torch.Tensor, N: int, K: int, out_dtype: torch.dtype = torch.bfloat16, *,
               out=None, workspace=None, a_block_size: int | None = None, stream=None) -> torch.Tensor:
    """Y = A B^T.  W4A4: a = packed u8 [M, K/2] with a_scales u8 [M, K/block] and a_tensor_scale
    (from nvfp4_quantize; both may be row-strided views of wider rows; the block size is
    a_block_size, else read from the scales' layout).  W4A16: a = bf16 [M, K], a_scales =
    a_tensor_scale = None."""
    M = a.shape[0]
    lda, ablk = _activation_pitch(mode, a, a_scales, a_block_size)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    ldc = out.stride(0)
    ws_need = nvfp4_gemm_workspace_bytes(mode, M, N, K, lda)
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_gemm_bs(mode, _ptr(a), _ptr(a_scales), _ptr(a_tensor_scale), ablk, _ptr(b_prepacked),
                             _ptr(b_tensor_scale), M, N, K, lda, _ptr(out), _dtype_code(out.dtype), ldc,
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_gemm_bs")
    return out


ACT_NONE, ACT_GELU_TANH = 0, 1


def nvfp4_gemm_requant_workspace_bytes(mode: int, M: int, N: int, K: int, lda: int | None = None) -> int:
    """Workspace bytes of nvfp4_gemm_requant for an activation with row pitch lda (K when None)."""
    return int(lib().nvfp4_gemm_requant_workspace_bytes_ld(mode, M, N, K, K if lda is None else lda))


def nvfp4_gemm_requant(mode: int, a: torch.Tensor, a_scales, a_tensor_scale, b_prepacked: torch.Tensor,
                       b_tensor_scale: torch.Tensor, N: int, K: int, out_tensor_scale: torch.Tensor, *,
                       bias=None, act: int = ACT_NONE, packed=None, scales=None, y=None, workspace=None,
                       a_block_size: int | None = None, stream=None):
    """NVFP4 output of A B^T (+ bias) (-> act) under the static out_tensor_scale (device fp32 [1]).
    Operands as nvfp4_gemm.  Returns (packed u8 [M, N/2], scales u8 [M, N/16]); when y (fp32 [M, >= N])
    is given it also receives the fp32 values that were quantized."""
    M = a.shape[0]
    lda, ablk = _activation_pitch(mode, a, a_scales, a_block_size)
    if packed is None:
        packed = torch.empty((M, N // 2), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty((M, N // 16), dtype=torch.uint8, device=a.device)
    ldy = 0 if y is None else y.stride(0)
    ws_need = nvfp4_gemm_requant_workspace_bytes(mode, M, N, K, lda)
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_gemm_requant_bs(mode, _ptr(a), _ptr(a_scales), _ptr(a_tensor_scale), ablk, _ptr(b_prepacked),
                                     _ptr(b_tensor_scale), M, N, K, lda, _ptr(bias), act, _ptr(out_tensor_scale),
                                     _ptr(packed), _ptr(scales), _ptr(y), ldy, _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check(st, "nvfp4_gemm_requant_bs")
    return packed, scales


# ---- MXFP4 (32-value blocks, E8M0 scales, no tensor scale) ------------------------------------

def nvfp4_mx_quantize(x: torch.Tensor, *, packed=None, scales=None, stream=None):
    """MXFP4-quantize x [M, K] (fp32 or bf16, K % 32 == 0).  Returns (packed u8 [M, K/2], scales u8 [M, K/32])."""
    M, K, ld = _rows(x, "x")
    if packed is None:
        packed = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, max(K // 32, 0)), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_mx_quantize(_ptr(x), _dtype_code(x.dtype), M, K, ld, _ptr(packed), _ptr(scales), _stream(stream)),
           "nvfp4_mx_quantize")
    return packed, scales


def nvfp4_mx_dequantize(packed: torch.Tensor, scales: torch.Tensor, dtype: torch.dtype = torch.float32, *, out=None,
                        stream=None) -> torch.Tensor:
    M, K = packed.shape[0], packed.shape[1] * 2
    if out is None:
        out = torch.empty((M, K), dtype=dtype, device=packed.device)
    _, _, ld = _rows(out, "out")
    _check(lib().nvfp4_mx_dequantize(_ptr(packed), _ptr(scales), M, K, _ptr(out), _dtype_code(out.dtype), ld,
                                     _stream(stream)), "nvfp4_mx_dequantize")
    return out


def nvfp4_mx_gemm(a: torch.Tensor, a_scales: torch.Tensor, b: torch.Tensor, b_scales: torch.Tensor,
                  out_dtype: torch.dtype = torch.bfloat16, *, out=None, stream=None) -> torch.Tensor:
    """Y = A B^T with A [M, K] and B [N, K] both canonical MXFP4 (packed codes + E8M0 scales)."""
    M, K = a.shape[0], a.shape[1] * 2
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check(lib().nvfp4_mx_gemm(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales), M, N, K, _ptr(out),
                               _dtype_code(out.dtype), out.stride(0), _stream(stream)), "nvfp4_mx_gemm")
    return out


__all__ = [
    "Status", "NVFP4Error", "lib", "LIB_PATH", "EXPORTED", "F32", "BF16", "W4A4", "W4A16",
    "SCALE_DYNAMIC", "SCALE_STATIC", "nvfp4_set_debug_checks",
    "nvfp4_quantize_workspace_bytes", "nvfp4_quantize", "nvfp4_quantize_noalloc", "nvfp4_dequantize",
    "nvfp4_fake_quantize",
    "FakeQuantizeSTE", "fake_quantize_ste",
    "nvfp4_prepacked_bytes", "nvfp4_prepack_weight", "nvfp4_unpack_weight",
    "nvfp4_gemm_workspace_bytes", "nvfp4_gemm",
    "ACT_NONE", "ACT_GELU_TANH", "nvfp4_gemm_requant_workspace_bytes", "nvfp4_gemm_requant",
    "nvfp4_mx_quantize", "nvfp4_mx_dequantize", "nvfp4_mx_gemm",
]
