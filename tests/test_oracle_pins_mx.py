"""Pins of the CPU oracle's MXFP4 functions against things other than itself (CPU only).

MXFP4 is named by the vllm-omni NVFP4 RFC (Motivation) as the related microscaling format but not
defined there; the definition followed is the public OCP Microscaling one: 32-value blocks sharing
an E8M0 scale X = 2^(b - 127) chosen so that amax / X lies in [4, 8) (b clamped to [0, 254],
b = 0 for an all-zero block), each value the E2M1 value nearest to v / X with ties to the even
code and clipping to +-6, sign copied, no tensor scale.

Pins: the scale rule as a property checked in exact rationals (not the oracle's frexp formula),
element codes by exhaustive search over the 16 codes in exact rationals, a hand-worked block,
the exact dequantized values, bf16 output against torch's cast, and a lossless on-grid round trip.
"""
import math
import random
from fractions import Fraction

import numpy as np
import torch

import oracle

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def brute_mx_byte(amax):
    """The byte b in [0, 254] with 4 <= amax / 2^(b-127) < 8, by search; 0 when none (tiny amax)."""
    if amax == 0:
        return 0
    a = Fraction(amax)
    for b in range(0, 255):
        X = Fraction(2) ** (b - 127)
        if 4 <= a / X < 8:
            return b
    assert a < 8 * Fraction(2) ** -127  # only tiny blocks have no such b: clamp to the smallest
    return 0


def brute_mx_code(v, byte):
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    x = abs(Fraction(v)) / (Fraction(2) ** (byte - 127))
    best, best_d = None, None
    for m, g in enumerate(GRID):
        d = abs(x - g)
        if best is None or d < best_d or (d == best_d and m % 2 == 0):
            best, best_d = m, d
    return sign | best


def test_mx_scale_byte_property():
    rng = random.Random(5)
    vals = [0.0, 1.0, 4.0, 6.0, 7.999, 8.0, 2.0 ** -126, 2.0 ** -130, 1e-45, 3.4e38, 2.0 ** 127]
    vals += [float(np.float32(rng.uniform(0.5, 1.0) * 2.0 ** rng.randint(-140, 127))) for _ in range(400)]
    vals += [float(np.nextafter(np.float32(2.0 ** k), np.float32(0))) for k in range(-120, 120, 7)]
    for a in vals:
        assert oracle.mx_scale_byte(a) == brute_mx_byte(a), a


def test_mx_element_codes_brute_force():
    for byte in (0, 1, 90, 125, 127, 130, 200, 252):
        X = 2.0 ** (byte - 127)
        for n in range(-520, 521, 1 if byte in (127, 125) else 7):
            with np.errstate(over="ignore"):
                v = float(np.float32(n / 64.0 * X))
            if not math.isfinite(v):
                continue  # beyond fp32 (only for the largest scale bytes)
            assert oracle.mx_element_code(v, byte) == brute_mx_code(v, byte), (byte, n)
    # fp32 neighbours of every decision boundary
    for byte in (100, 127, 140):
        X = Fraction(2) ** (byte - 127)
        for t in (Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4), Fraction(5, 2), Fraction(7, 2),
                  Fraction(5), Fraction(6), Fraction(7)):
            c = np.float32(float(t * X))
            for d in range(-4, 5):
                v = float((c.view(np.uint32) + np.uint32(d % (1 << 32)) if d >= 0 else c.view(np.uint32) - np.uint32(-d)).view(np.float32))
                for sv in (v, -v):
                    assert oracle.mx_element_code(sv, byte) == brute_mx_code(sv, byte), (byte, t, d)


def test_mx_worked_block():
    """Hand-worked block: amax = 7 gives floor(log2 7) = 2, X = 1 (byte 127).  Ties go to the even
    code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0;
    7 clips to 6; -0.1 rounds to -0 (code 8)."""
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.1, -0.0, 0.0, -6.0, 3.0, -1.5, 0.5, 4.5]
    want = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x7, 0x8, 0x8, 0x0, 0xF, 0x5, 0xB, 0x1, 0x6]
    x = np.array([vals + vals], dtype=np.float32)
    p, s = oracle.mx_quantize(x)
    assert s.tolist() == [[127]]
    codes = [(p[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(32)]
    assert codes == want + want


def test_mx_quantize_brute_force_tiny():
    rng = np.random.default_rng(9)
    for trial in range(5):
        M, K = int(rng.integers(1, 4)), 32 * int(rng.integers(1, 4))
        x = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        if trial == 2:
            x[:, :32] = 0.0
        p, s = oracle.mx_quantize(x)
        for i in range(M):
            for j in range(K // 32):
                blk = [float(v) for v in x[i, 32 * j:32 * j + 32]]
                b = brute_mx_byte(max(abs(v) for v in blk))
                assert s[i, j] == b
                for t in range(32):
                    c = (p[i, 16 * j + t // 2] >> (4 * (t % 2))) & 15
                    assert c == brute_mx_code(blk[t], b)


def test_mx_dequantize_exact_and_bf16_cast():
    rng = np.random.default_rng(2)
    M, K = 3, 64
    p = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    s = rng.integers(0, 253, (M, K // 32), dtype=np.uint8)  # the bytes the quantizer can produce
    s[0, 0] = 0
    s[1, 0] = 252
    y32, y16 = oracle.mx_dequantize(p, s)
    for i in range(M):
        for k in range(K):
            c = (p[i, k // 2] >> (4 * (k % 2))) & 15
            q = GRID[c & 7] * (-1 if c & 8 else 1)
            want = q * Fraction(2) ** (int(s[i, k // 32]) - 127)
            if want != 0:
                assert Fraction(float(y32[i, k])) == want
            else:
                assert y32[i, k] == 0.0 and math.copysign(1.0, float(y32[i, k])) == (-1.0 if c & 8 else 1.0)
    t16 = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y16, t16)
    # byte 254 (never produced by the quantizer): 6 * 2^127 rounds to +-inf in fp32
    y, _ = oracle.mx_dequantize(np.array([[0x7F] * 16], np.uint8), np.array([[254]], np.uint8))
    assert np.isinf(y[0, 0]) and y[0, 0] < 0 and np.isinf(y[0, 1]) and y[0, 1] > 0  # low nibble 15 = -6


def test_mx_round_trip_on_grid():
    """Blocks whose values are grid points times X with a block maximum in [4X, 6X] come back
    unchanged."""
    rng = np.random.default_rng(4)
    for b in (60, 127, 180):
        X = 2.0 ** (b - 127)
        v = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(4, 64)) * X
        v[:, 0] = 4 * X
        v[:, 32] = -6 * X
        x = v.astype(np.float32)
        p, s = oracle.mx_quantize(x)
        assert (s == b).all()
        y32, _ = oracle.mx_dequantize(p, s)
        np.testing.assert_array_equal(y32, x)
