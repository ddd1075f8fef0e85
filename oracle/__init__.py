"""CPU oracle for NVFP4 quantization and the dequantize-then-matmul GEMM (numpy + ctypes).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product library (``nvfp4_quantized_gemm_amd``)
never imports it and shares no code with it; the C source it wraps, ``nvfp4_oracle.c``, states
the definitions and the readings of the pages that it follows.

Arrays:
  * fp32 inputs are ``np.float32``; bfloat16 inputs are their bit patterns as ``np.uint16``.
  * ``packed`` is ``uint8 [M, K/2]`` (element 2i in the low nibble of byte i),
    ``scales`` is ``uint8 [M, K/16]`` (OCP E4M3FN bytes), ``S`` is an ``np.float32``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_nvfp4.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ora_e2m1_value.restype = ctypes.c_double
    lib.ora_e2m1_value.argtypes = [ctypes.c_int]
    lib.ora_e4m3_value.restype = ctypes.c_double
    lib.ora_e4m3_value.argtypes = [ctypes.c_int]
    lib.ora_bf16_round.restype = ctypes.c_uint16
    lib.ora_bf16_round.argtypes = [ctypes.c_float]
    lib.ora_tensor_scale.restype = ctypes.c_int
    lib.ora_tensor_scale.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_float)]
    lib.ora_block_scale_byte.restype = ctypes.c_int
    lib.ora_block_scale_byte.argtypes = [ctypes.c_double, ctypes.c_float]
    lib.ora_element_code.restype = ctypes.c_int
    lib.ora_element_code.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_float]
    lib.ora_quantize.restype = ctypes.c_int
    lib.ora_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _vp, _vp, ctypes.c_int]
    lib.ora_dequantize.restype = ctypes.c_int
    lib.ora_dequantize.argtypes = [_vp, _vp, ctypes.c_float, _i64, _i64, _vp, _vp, ctypes.c_int]
    lib.ora_quantize_bs.restype = ctypes.c_int
    lib.ora_quantize_bs.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, _vp, _vp,
                                    ctypes.c_int]
    lib.ora_dequantize_bs.restype = ctypes.c_int
    lib.ora_dequantize_bs.argtypes = [_vp, _vp, ctypes.c_float, _i64, _i64, ctypes.c_int, _vp, _vp, ctypes.c_int]
    lib.ora_mx_scale_byte.restype = ctypes.c_int
    lib.ora_mx_scale_byte.argtypes = [ctypes.c_double]
    lib.ora_mx_element_code.restype = ctypes.c_int
    lib.ora_mx_element_code.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.ora_mx_quantize.restype = ctypes.c_int
    lib.ora_mx_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, ctypes.c_int]
    lib.ora_mx_dequantize.restype = ctypes.c_int
    lib.ora_mx_dequantize.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, ctypes.c_int]
    lib.ora_gemm.restype = ctypes.c_int
    lib.ora_gemm.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, ctypes.c_int]
    lib.ora_gemm_sampled.restype = ctypes.c_int
    lib.ora_gemm_sampled.argtypes = [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp]
    _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _x_args(x: np.ndarray):
    if x.dtype == np.float32:
        dtype = 0
    elif x.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("oracle inputs are float32 or bfloat16 bit patterns (uint16)")
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.size == 0:  # empty: no element is read
        return dtype, x.shape[0], x.shape[1], x.shape[1]
    if x.strides[1] != x.itemsize:
        raise ValueError("expected a 2-D array with unit stride along K")
    ld = x.strides[0] // x.itemsize
    return dtype, x.shape[0], x.shape[1], ld


# ---- scalar helpers -------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().ora_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().ora_e4m3_value(int(byte))


def bf16_round(y: float) -> int:
    return int(_load().ora_bf16_round(float(np.float32(y))))


def block_scale_byte(amax: float, S) -> int:
    return _load().ora_block_scale_byte(float(amax), float(np.float32(S)))


def element_code(v, byte: int, S) -> int:
    return _load().ora_element_code(float(np.float32(v)), int(byte), float(np.float32(S)))


# ---- array operations ------------------------------------------------------------------------

def tensor_scale(x: np.ndarray) -> np.float32:
    """Dynamic per-tensor scale S = RN32(max|x| / 2688)."""
    dtype, M, K, ld = _x_args(x)
    out = ctypes.c_float(0.0)
    if _load().ora_tensor_scale(_ptr(x), dtype, M, K, ld, ctypes.byref(out)) != 0:
        raise ValueError("non-finite input")
    return np.float32(out.value)


BLOCK_SIZES = (1, 2, 4, 8, 16, 32, 64)  # NVFP4-DiT page, Algorithm 1 / Eq. 9


def quantize(x: np.ndarray, S=None, threads: int | None = None, block: int = 16):
    """Quantize x [M, K] (K % block == 0, K even).  S=None: dynamic scale; else the given static scale.
    `block` is the number of consecutive values along K sharing one E4M3 scale byte.

    Returns (packed uint8 [M, K/2], scales uint8 [M, K/block], S float32).
    """
    dtype, M, K, ld = _x_args(x)
    if block not in BLOCK_SIZES or K % block or K % 2:
        raise ValueError("K must be a multiple of the block size (and even)")
    if S is None:
        S = tensor_scale(x)
    S = np.float32(S)
    packed = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // block), np.uint8)
    if block == 16:
        rc = _load().ora_quantize(_ptr(x), dtype, M, K, ld, float(S), _ptr(packed), _ptr(scales),
                                  threads or default_threads())
    else:
        rc = _load().ora_quantize_bs(_ptr(x), dtype, M, K, ld, float(S), block, _ptr(packed), _ptr(scales),
                                     threads or default_threads())
    if rc != 0:
        raise ValueError("precondition failed (non-finite input or invalid S)")
    return packed, scales, S


def dequantize(packed: np.ndarray, scales: np.ndarray, S, threads: int | None = None):
    """Returns (y_f32 float32 [M, K], y_bf16 uint16 [M, K]); the block size is K / scales.shape[1]."""
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    M, K = packed.shape[0], packed.shape[1] * 2
    if scales.shape[0] != M or scales.shape[1] == 0 or K % scales.shape[1]:
        raise ValueError("scales shape does not match packed")
    block = K // scales.shape[1]
    y32 = np.empty((M, K), np.float32)
    y16 = np.empty((M, K), np.uint16)
    if block == 16:
        rc = _load().ora_dequantize(_ptr(packed), _ptr(scales), float(np.float32(S)), M, K, _ptr(y32), _ptr(y16),
                                    threads or default_threads())
    else:
        rc = _load().ora_dequantize_bs(_ptr(packed), _ptr(scales), float(np.float32(S)), M, K, block, _ptr(y32),
                                       _ptr(y16), threads or default_threads())
    if rc != 0:
        raise ValueError("precondition failed")
    return y32, y16


# ---- MXFP4 (OCP microscaling: 32-value blocks, E8M0 scales, no tensor scale) ---------------------

def mx_scale_byte(amax: float) -> int:
    return _load().ora_mx_scale_byte(float(amax))


def mx_element_code(v, byte: int) -> int:
    return _load().ora_mx_element_code(float(np.float32(v)), int(byte))


def mx_quantize(x: np.ndarray, threads: int | None = None):
    """MXFP4-quantize x [M, K] (K % 32 == 0).  Returns (packed uint8 [M, K/2], scales uint8 [M, K/32])."""
    dtype, M, K, ld = _x_args(x)
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    packed = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 32), np.uint8)
    rc = _load().ora_mx_quantize(_ptr(x), dtype, M, K, ld, _ptr(packed), _ptr(scales), threads or default_threads())
    if rc != 0:
        raise ValueError("precondition failed (non-finite input)")
    return packed, scales


def mx_dequantize(packed: np.ndarray, scales: np.ndarray, threads: int | None = None):
    """Returns (y_f32 float32 [M, K], y_bf16 uint16 [M, K])."""
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    M, K = packed.shape[0], packed.shape[1] * 2
    if scales.shape != (M, K // 32):
        raise ValueError("scales shape does not match packed")
    y32 = np.empty((M, K), np.float32)
    y16 = np.empty((M, K), np.uint16)
    rc = _load().ora_mx_dequantize(_ptr(packed), _ptr(scales), M, K, _ptr(y32), _ptr(y16), threads or default_threads())
    if rc != 0:
        raise ValueError("precondition failed")
    return y32, y16


def gemm(A: np.ndarray, B: np.ndarray, threads: int | None = None):
    """Y = A @ B^T in fp64 accumulation of fp32 operands; also R = |A| @ |B|^T (elementwise sums)."""
    A = np.ascontiguousarray(A, np.float32)
    B = np.ascontiguousarray(B, np.float32)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    Y = np.empty((M, N), np.float64)
    R = np.empty((M, N), np.float64)
    _load().ora_gemm(_ptr(A), K, _ptr(B), K, M, N, K, _ptr(Y), _ptr(R), threads or default_threads())
    return Y, R


def gemm_sampled(A: np.ndarray, B: np.ndarray, rows, cols):
    """Y and R at the output positions (rows[t], cols[t])."""
    A = np.ascontiguousarray(A, np.float32)
    B = np.ascontiguousarray(B, np.float32)
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    K = A.shape[1]
    if B.shape[1] != K or rows.shape != cols.shape:
        raise ValueError("shape mismatch")
    Y = np.empty(rows.shape, np.float64)
    R = np.empty(rows.shape, np.float64)
    _load().ora_gemm_sampled(_ptr(A), K, _ptr(B), K, K, _ptr(rows), _ptr(cols), rows.size, _ptr(Y), _ptr(R))
    return Y, R


def bf16_to_f32(x16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (no arithmetic of the method)."""
    return (x16.astype(np.uint32) << 16).view(np.float32)


# ---- linear-layer epilogue before requantization ------------------------------------------------
# The GEMM with NVFP4 output forms y = Y (+ bias[n]) (-> activation) and quantizes y under a static
# tensor scale with the rules of `quantize` [NVFP4-DiT page, Methodology section 3: operands of the
# next W4A4 product; Definition III.1: the encoding].  The pages name no activation; the tanh form
# of GELU (the DiT-family MLP activation) is the reading taken.

def gelu_tanh(x) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x * x * x)))


def linear_epilogue(Y: np.ndarray, bias=None, act: int = 0) -> np.ndarray:
    """y = Y + bias (per output column, fp64) followed by the activation (0: none, 1: GELU tanh)."""
    y = np.asarray(Y, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if act == 1:
        y = gelu_tanh(y)
    elif act != 0:
        raise ValueError("unknown activation")
    return y
