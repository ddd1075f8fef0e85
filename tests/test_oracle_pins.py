"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins the oracle to: a brute-force search in exact rational arithmetic,
a library routine (torch's float8_e4m3fn / bfloat16 casts, fp64 matmul), hand-worked blocks
(tests/golden/worked_blocks.json), closed forms, or invariants of the definition.
Definition followed: Q_FP4(v; s) = s * clip(round(v/s)_FP4, -6, 6) [NVFP4-DiT page, Methodology
section 1, Definition III.1] with s = e * S, e an E4M3 scale per 16 values and S an fp32 tensor
scale [vllm-omni NVFP4 RFC, Motivation].
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.json")

# ---------------------------------------------------------------------------------------------
# independent brute-force helpers (exact rationals; they do not call the oracle)

E2M1_STATED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the grid the format's bits imply


def _e4m3_from_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    return [float(v) for v in b]


E4M3_TORCH = _e4m3_from_torch()
E4M3_POS = [(i, Fraction(E4M3_TORCH[i])) for i in range(0x7F)]  # bytes 0x00..0x7E


def brute_scale_byte(amax, S):
    """Nearest E4M3 byte (0..0x7E) to amax/(6S) in exact rationals, ties to even byte."""
    if amax == 0:
        return 0
    r = Fraction(amax) / (6 * Fraction(S))
    best, best_d = None, None
    for b, v in E4M3_POS:
        d = abs(r - v)
        if best is None or d < best_d or (d == best_d and b % 2 == 0):
            best, best_d = b, d
    return best


def brute_code(v, byte, S):
    """Nearest signed E2M1 code of v/(e S) in exact rationals, ties to even code, clip to +-6."""
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    e = Fraction(E4M3_TORCH[byte])
    if e == 0:
        return sign
    x = abs(Fraction(v)) / (e * Fraction(S))
    best, best_d = None, None
    for m, g in enumerate(E2M1_STATED):
        d = abs(x - Fraction(g))
        if best is None or d < best_d or (d == best_d and m % 2 == 0):
            best, best_d = m, d
    return sign | best


def brute_quantize(x32, S):
    """Whole quantizer on a tiny fp32 array, built from the brute-force pieces."""
    M, K = x32.shape
    packed = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    for i in range(M):
        for j in range(K // 16):
            blk = [float(v) for v in x32[i, 16 * j:16 * j + 16]]
            byte = brute_scale_byte(max(abs(v) for v in blk), S)
            scales[i, j] = byte
            for t in range(0, 16, 2):
                c0 = brute_code(blk[t], byte, S)
                c1 = brute_code(blk[t + 1], byte, S)
                packed[i, 8 * j + t // 2] = c0 | (c1 << 4)
    return packed, scales


def f32(v):
    return np.float32(v)


def f32_bits(v):
    return int(np.float32(v).view(np.uint32))


def from_bits(b):
    return float(np.uint32(b).view(np.float32))


def _parse(v):
    if isinstance(v, str):
        return float(v)
    return float(v)


# ---------------------------------------------------------------------------------------------
# element format


def test_e2m1_grid_is_the_bit_format_grid():
    """Codes 0..7 give the grid {0, .5, 1, 1.5, 2, 3, 4, 6}; 8..15 their negatives (8 = -0)."""
    pos = [oracle.e2m1_value(c) for c in range(8)]
    assert pos == E2M1_STATED
    for c in range(8):
        neg = oracle.e2m1_value(c + 8)
        assert neg == -pos[c]
        assert math.copysign(1.0, neg) == -1.0


def test_e4m3_decode_matches_torch_all_bytes():
    for b in range(256):
        ours, ref = oracle.e4m3_value(b), E4M3_TORCH[b]
        if math.isnan(ref):
            assert math.isnan(ours), hex(b)
        else:
            assert ours == ref and math.copysign(1, ours) == math.copysign(1, ref), hex(b)
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


# ---------------------------------------------------------------------------------------------
# block scale (E4M3 encode)


def test_block_scale_matches_torch_fp8_cast():
    """With S = 2^k and amax = r * 6 * S exact, the byte equals torch's RNE cast of min(r, 448)."""
    rng = random.Random(11)
    rs = []
    for _ in range(4000):
        r = f32(2.0 ** rng.uniform(-12, 9.5))
        r = from_bits(f32_bits(r) & ~0x3)  # <= 22 significant bits so 3 r is exact
        rs.append(r)
    vals = [v for _, v in E4M3_POS]
    for a, b in zip(vals[:-1], vals[1:]):
        rs.append(float((a + b) / 2))  # exact midpoints: ties
    rs += [2.0 ** -10, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 7.5 * 2 ** -9, 448.0, 460.0, 464.0, 470.0, 1e4]
    for r in rs:
        k = rng.randint(-30, 10)
        S = 2.0 ** k
        amax = r * 6.0 * S
        assert float(f32(amax)) == amax
        ref = torch.tensor([min(r, 448.0)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
        assert oracle.block_scale_byte(amax, S) == ref, (r, k)


def test_block_scale_brute_force_generic_S():
    """Generic (non power-of-two) S and random amax against exact-rational nearest search."""
    rng = random.Random(5)
    for _ in range(3000):
        S = f32(rng.uniform(0.5, 1.0) * 2.0 ** rng.randint(-40, 20))
        amax = f32(float(S) * 6 * 2.0 ** rng.uniform(-13, 10))
        assert oracle.block_scale_byte(float(amax), S) == brute_scale_byte(float(amax), float(S))


def test_block_scale_constructed_ties_generic_S():
    """amax exactly on an E4M3 midpoint times 6S, with S having few significant bits."""
    vals = [v for _, v in E4M3_POS]
    rng = random.Random(9)
    n = 0
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        S = Fraction(rng.choice([3, 5, 7, 11, 13])) * Fraction(2) ** rng.randint(-20, 0)
        amax = mid * 6 * S
        if float(f32(float(amax))) != amax:
            continue
        n += 1
        ours = oracle.block_scale_byte(float(amax), float(S))
        assert ours == brute_scale_byte(float(amax), float(S))
        assert ours % 2 == 0
    assert n > 100


# ---------------------------------------------------------------------------------------------
# element rounding


def test_element_codes_grid_of_sixty_fourths():
    """Every multiple of 1/64 in [-8, 8] (in units of eS), for several scales, vs brute force."""
    for byte, S in [(0x38, 1.0), (0x7E, 2.0 ** -9), (0x03, 2.0 ** -4), (0x45, 0.75), (0x08, 3.0)]:
        es = E4M3_TORCH[byte] * S
        for n in range(-512, 513):
            v = n / 64.0 * es
            assert float(f32(v)) == v
            assert oracle.element_code(v, byte, S) == brute_code(v, byte, S), (byte, S, n)


def test_element_codes_near_every_threshold():
    """fp32 neighbours (+-6 ulps) of every decision boundary t e S, generic S, vs brute force."""
    rng = random.Random(3)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    for _ in range(60):
        byte = rng.randint(1, 0x7E)
        S = f32(rng.uniform(0.5, 1.0) * 2.0 ** rng.randint(-30, 10))
        es = Fraction(E4M3_TORCH[byte]) * Fraction(float(S))
        for t in ties:
            c = f32(float(t * es))
            for d in range(-6, 7):
                v = from_bits(f32_bits(c) + d)
                for sv in (v, -v):
                    assert oracle.element_code(sv, byte, S) == brute_code(sv, byte, float(S))


def test_element_sign_of_zero_and_flushed_blocks():
    assert oracle.element_code(-0.0, 0x38, 1.0) == 8
    assert oracle.element_code(0.0, 0x38, 1.0) == 0
    assert oracle.element_code(-0.1, 0x38, 1.0) == 8  # rounds to zero, keeps the sign
    assert oracle.element_code(-3.0, 0x00, 1.0) == 8  # flushed block
    assert oracle.element_code(100.0, 0x38, 1.0) == 7  # clipped to 6


def test_whole_quantizer_brute_force_tiny():
    """Small random tensors (several rows and blocks) against the brute-force quantizer."""
    rng = np.random.default_rng(17)
    for trial in range(6):
        M, K = rng.integers(1, 4), 16 * rng.integers(1, 4)
        x = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial == 3:
            x[:, :16] = 0.0
        S = oracle.tensor_scale(x)
        p, s, S2 = oracle.quantize(x)
        assert S2 == S
        bp, bs = brute_quantize(x, float(S))
        np.testing.assert_array_equal(s, bs)
        np.testing.assert_array_equal(p, bp)


# ---------------------------------------------------------------------------------------------
# tensor scale


def test_tensor_scale_closed_form():
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = (rng.standard_normal((3, 32)) * 10.0 ** rng.uniform(-5, 5)).astype(np.float32)
        amax = np.float32(np.abs(x).max())
        assert oracle.tensor_scale(x) == np.float32(amax / np.float32(2688.0))
    assert f32_bits(oracle.tensor_scale(np.ones((1, 16), np.float32))) == 0x39C30C31
    assert oracle.tensor_scale(np.full((1, 16), 5.25, np.float32)) == 2.0 ** -9
    assert oracle.tensor_scale(np.full((1, 16), -10.5, np.float32)) == 2.0 ** -8


def test_tensor_scale_and_quantize_respect_row_stride():
    rng = np.random.default_rng(2)
    big = rng.standard_normal((4, 64)).astype(np.float32)
    big[:, 48:] = 1000.0  # padding beyond K must be ignored
    view = big[:, :48]
    assert oracle.tensor_scale(view) == oracle.tensor_scale(np.ascontiguousarray(view))
    p1, s1, _ = oracle.quantize(view)
    p2, s2, _ = oracle.quantize(np.ascontiguousarray(view))
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------------------------------------
# hand-worked blocks


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_worked_blocks(case):
    x = np.array([_parse(v) for v in case["x"]], np.float32).reshape(case["M"], case["K"])
    p, s, S = oracle.quantize(x)
    assert f32_bits(S) == int(case["S_bits"], 16)
    assert [int(v) for v in s.ravel()] == [int(h, 16) for h in case["scales"]]
    y32, y16 = oracle.dequantize(p, s, S)
    if "packed" in case:
        assert [int(v) for v in p.ravel()] == [int(h, 16) for h in case["packed"]]
        exp = np.array([_parse(v) for v in case["dequant"]], np.float32)
        np.testing.assert_array_equal(y32.ravel(), exp)
        assert list(np.signbit(y32.ravel())) == list(np.signbit(exp))
    else:
        assert int(p[0, 8]) == int(case["packed_block1_first_byte"], 16)
        exp = np.array([_parse(v) for v in case["dequant_block1_first_two"]], np.float32)
        np.testing.assert_array_equal(y32[0, 16:18], exp)
        assert list(np.signbit(y32[0, 16:18])) == list(np.signbit(exp))


def test_worked_requantize_counterexample():
    g = _golden()["requantize"]
    x = np.array(g["x"], np.float32).reshape(1, 16)
    _, s, _ = oracle.quantize(x, S=g["S"])
    assert int(s[0, 0]) == int(g["scales"][0], 16)


def test_worked_gemm_k16():
    cases = {c["name"]: c for c in _golden()["cases"]}
    a = np.array([_parse(v) for v in cases["tie_block"]["dequant"]], np.float32).reshape(1, 16)
    b = np.array(cases["all_equal_block"]["dequant"], np.float32).reshape(1, 16)
    Y, R = oracle.gemm(a, b)
    g = _golden()["gemm"]
    assert Y[0, 0] == g["y"] and R[0, 0] == g["R"]


# ---------------------------------------------------------------------------------------------
# dequantize


def test_dequant_single_rounding_brute_force():
    """y32 is the fp32 nearest (ties to even) to the exact rational q e S: checked by exact search."""
    rng = np.random.default_rng(4)
    packed = rng.integers(0, 256, (3, 16), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (3, 2), dtype=np.uint8)
    S = np.float32(0.3711)
    y32, _ = oracle.dequantize(packed, scales, S)
    for i in range(3):
        for k in range(32):
            code = (int(packed[i, k // 2]) >> (4 * (k % 2))) & 15
            exact = Fraction(E2M1_STATED[code & 7]) * Fraction(E4M3_TORCH[scales[i, k // 16]]) * Fraction(float(S))
            if code & 8:
                exact = -exact
            y = float(y32[i, k])
            lo = np.nextafter(np.float32(y), np.float32(-np.inf))
            hi = np.nextafter(np.float32(y), np.float32(np.inf))
            d = abs(Fraction(y) - exact)
            assert d <= abs(Fraction(float(lo)) - exact) and d <= abs(Fraction(float(hi)) - exact)
            if code >= 8:
                assert np.signbit(y32[i, k])


def test_dequant_bf16_matches_torch_rounding():
    rng = np.random.default_rng(6)
    packed = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (8, 8), dtype=np.uint8)
    y32, y16 = oracle.dequantize(packed, scales, np.float32(0.0123))
    ref = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y16, ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(8)
    xs = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)
    ties = (rng.integers(0, 2 ** 15, 2000).astype(np.uint32) << 16) | 0x8000
    xs = np.concatenate([xs, ties.view(np.float32)])
    xs = xs[np.isfinite(xs)]
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_round(v) for v in xs], np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_lossless_round_trip_on_grid():
    """Values already on the grid (each block holding a +-6 e S maximum, S = 2^-8) round-trip."""
    rng = np.random.default_rng(12)
    M, K = 4, 64
    S = 2.0 ** -8
    x = np.zeros((M, K), np.float32)
    bytes_ = rng.integers(1, 0x7F, (M, K // 16))
    for i in range(M):
        for j in range(K // 16):
            e = E4M3_TORCH[bytes_[i, j]]
            codes = rng.integers(0, 16, 16)
            codes[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
            vals = [math.copysign(E2M1_STATED[c & 7], -1.0 if c & 8 else 1.0) * e * S for c in codes]
            x[i, 16 * j:16 * j + 16] = vals
    p, s, _ = oracle.quantize(x, S=S)
    np.testing.assert_array_equal(s, bytes_)
    y32, _ = oracle.dequantize(p, s, np.float32(S))
    np.testing.assert_array_equal(y32, x)
    assert (np.signbit(y32) == np.signbit(x)).all()


# ---------------------------------------------------------------------------------------------
# invariants of the definition


def _random_blocks(rng, n):
    """Blocks mixing scales, exact zeros, negative zeros and outliers."""
    x = rng.standard_normal((n, 16)) * 10.0 ** rng.uniform(-6, 4, (n, 1))
    x[rng.random((n, 16)) < 0.05] = 0.0
    x[rng.random((n, 16)) < 0.02] = -0.0
    x[::7] *= rng.choice([1.0, 50.0], size=(len(x[::7]), 16))
    return x.astype(np.float32).reshape(1, -1)


def test_invariants_random():
    rng = np.random.default_rng(21)
    x = _random_blocks(rng, 3000)
    p, s, S = oracle.quantize(x)
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(x.shape)
    mags = codes & 7
    y32, _ = oracle.dequantize(p, s, S)
    S = float(S)
    xb = x.reshape(-1, 16)
    mb = mags.reshape(-1, 16)
    sb = s.reshape(-1)
    assert (sb <= 0x7E).all()
    # sign copied from the input, including -0.0
    assert ((codes >> 3).astype(bool) == np.signbit(x)).all()
    for j in range(xb.shape[0]):
        e = E4M3_TORCH[sb[j]]
        blk = np.abs(xb[j].astype(np.float64))
        if blk.max() == 0:
            assert sb[j] == 0
        if sb[j] >= 3:
            assert mb[j].max() == 7
        # monotone within a block
        order = np.argsort(blk, kind="stable")
        assert (np.diff(mb[j][order]) >= 0).all()
        # |Q(v)| <= 6 e S
        assert (np.abs(y32.reshape(-1, 16)[j]) <= 6 * e * S * (1 + 2 ** -23)).all()


def test_error_bound_half_ulp_reading():
    """For in-range values (e > 0, 1 <= |v|/(eS) <= 6): |Q(v) - v| <= 2^-3 * 2^(floor(log2 x)+1) * e S.

    This is the reading of Lemma III.2's epsilon = 2^-3 that holds (half an E2M1 step relative to
    the top of the value's binade); the literal per-element relative reading fails, e.g. x = 5 -> 4.
    """
    rng = np.random.default_rng(31)
    x = _random_blocks(rng, 4000)
    p, s, S = oracle.quantize(x)
    y32, _ = oracle.dequantize(p, s, S)
    S = float(S)
    e = np.array([E4M3_TORCH[b] for b in s.ravel()]).repeat(16)
    v = x.ravel().astype(np.float64)
    y = y32.ravel().astype(np.float64)
    es = e * S
    ok = es > 0
    xs = np.where(ok, np.abs(v) / np.where(ok, es, 1), 0)
    inr = ok & (xs >= 1) & (xs <= 6)
    bound = 2.0 ** -3 * 2.0 ** (np.floor(np.log2(np.where(inr, xs, 1))) + 1) * es
    err = np.abs(y - v)
    # fp32 rounding of the dequantized value adds at most half an fp32 ulp of |y|
    assert (err[inr] <= bound[inr] + np.abs(y[inr]) * 2 ** -24).all()
    assert (err[ok & (xs < 1)] <= 0.25 * es[ok & (xs < 1)] * (1 + 2 ** -20)).all()
    literal = np.abs(err[inr]) > 0.125 * np.abs(v[inr])
    assert literal.any()  # the literal per-element relative reading is violated


def test_literal_epsilon_counterexample():
    S = 2.0 ** -9  # e S = 0.875 with byte 0x7E
    v = 5 * 0.875
    c = oracle.element_code(v, 0x7E, S)
    assert c == 6  # value 4: relative error 0.2 > 2^-3
    assert abs(4 - 5) / 5 > 0.125


def test_requantize_idempotent_for_scale_bytes_0_or_ge_3():
    rng = np.random.default_rng(41)
    x = _random_blocks(rng, 4000)
    S = oracle.tensor_scale(x)
    p, s, _ = oracle.quantize(x, S=S)
    y32, y16 = oracle.dequantize(p, s, S)
    for y in (y32, oracle.bf16_to_f32(y16)):
        p2, s2, _ = oracle.quantize(np.ascontiguousarray(y), S=S)
        keep = (s.ravel() == 0) | (s.ravel() >= 3)
        np.testing.assert_array_equal(s2.ravel()[keep], s.ravel()[keep])
        pb = p.reshape(-1, 8)[keep]
        p2b = p2.reshape(-1, 8)[keep]
        np.testing.assert_array_equal(p2b, pb)


def test_requantize_dynamic_scale_stable():
    rng = np.random.default_rng(43)
    x = _random_blocks(rng, 500)
    p, s, S = oracle.quantize(x)
    y32, _ = oracle.dequantize(p, s, S)
    S2 = oracle.tensor_scale(y32)
    assert abs(float(S2) - float(S)) <= float(np.spacing(np.float32(S)))


def test_memory_ratio_closed_form():
    """0.5 B of codes + 1/16 B of scale per element: 2/0.5625 ~ 3.56x vs FP16, 1/0.5625 ~ 1.78x vs FP8
    (the ~3.5x / ~1.8x of the vllm-omni RFC, Motivation)."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    p, s, _ = oracle.quantize(x)
    per_elem = (p.nbytes + s.nbytes) / x.size
    assert per_elem == 0.5625
    assert round(2 / per_elem, 2) == 3.56 and round(1 / per_elem, 2) == 1.78


# ---------------------------------------------------------------------------------------------
# GEMM


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 48), (17, 9, 160), (64, 33, 512)])
def test_gemm_matches_fp64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    xa = rng.standard_normal((M, K)).astype(np.float32)
    xb = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    pa, sa, Sa = oracle.quantize(xa)
    pb, sb, Sb = oracle.quantize(xb)
    A, _ = oracle.dequantize(pa, sa, Sa)
    B, _ = oracle.dequantize(pb, sb, Sb)
    Y, R = oracle.gemm(A, B)
    At, Bt = torch.from_numpy(A).double(), torch.from_numpy(B).double()
    ref = (At @ Bt.T).numpy()
    refR = (At.abs() @ Bt.abs().T).numpy()
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * (refR.max() + 1))
    np.testing.assert_allclose(R, refR, rtol=1e-13)
    rows = rng.integers(0, M, 20)
    cols = rng.integers(0, N, 20)
    Ys, Rs = oracle.gemm_sampled(A, B, rows, cols)
    np.testing.assert_array_equal(Ys, Y[rows, cols])
    np.testing.assert_array_equal(Rs, R[rows, cols])


def test_gemm_lossless_on_grid_and_zero():
    """On-grid operands: the GEMM of dequantized values equals the exact matmul of the raw inputs."""
    rng = np.random.default_rng(13)
    S = 2.0 ** -4
    def on_grid(n, k):
        codes = rng.integers(0, 16, (n, k))
        codes[:, ::16] = 7
        v = np.array(E2M1_STATED)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
        return (v * E4M3_TORCH[0x30] * S).astype(np.float32)
    xa, xb = on_grid(5, 64), on_grid(7, 64)
    pa, sa, _ = oracle.quantize(xa, S=S)
    pb, sb, _ = oracle.quantize(xb, S=S)
    A, _ = oracle.dequantize(pa, sa, S)
    B, _ = oracle.dequantize(pb, sb, S)
    Y, _ = oracle.gemm(A, B)
    np.testing.assert_array_equal(Y, xa.astype(np.float64) @ xb.astype(np.float64).T)
    Z, RZ = oracle.gemm(np.zeros((2, 32), np.float32), B[:, :32])
    assert (Z == 0).all() and (RZ == 0).all()


# ---------------------------------------------------------------------------------------------
# bf16 inputs


def test_bf16_input_equals_fp32_of_same_values():
    rng = np.random.default_rng(51)
    x32 = rng.standard_normal((5, 96)).astype(np.float32)
    x16 = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    widened = oracle.bf16_to_f32(x16)
    p1, s1, S1 = oracle.quantize(x16)
    p2, s2, S2 = oracle.quantize(widened)
    assert S1 == S2
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)


# ---- linear epilogue (GELU, bias) of the NVFP4-output GEMM ---------------------------------------

def test_gelu_tanh_matches_torch_and_identities():
    """Pinned by torch's own tanh-form GELU in fp64 (library routine) and by two closed forms:
    g(x) - g(-x) = x exactly for this form (the tanh terms cancel), and g(0) = 0."""
    g = torch.Generator().manual_seed(17)
    x = torch.cat([torch.randn(4096, generator=g, dtype=torch.float64) * 4,
                   torch.tensor([0.0, -0.0, 1e-300, -1e-300, 3.0, -3.0, 40.0, -40.0], dtype=torch.float64)])
    ours = oracle.gelu_tanh(x.numpy())
    ref = torch.nn.functional.gelu(x, approximate="tanh").numpy()
    # for large negative x both forms lose relative accuracy to the cancellation in 1 + tanh(u),
    # so the bound is relative to |g| plus a few ulps of |x|
    xa = np.abs(x.numpy())
    assert np.all(np.abs(ours - ref) <= 1e-14 * np.abs(ref) + 4e-16 * xa)
    assert np.all(np.abs((ours - oracle.gelu_tanh(-x.numpy())) - x.numpy()) <= 4e-16 * xa)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(40.0) == 40.0 and abs(oracle.gelu_tanh(-40.0)) < 1e-300 + 1e-12


def test_linear_epilogue_bias_per_column():
    Y = np.arange(12, dtype=np.float64).reshape(3, 4)
    b = np.array([1.0, -2.0, 0.5, 0.0])
    np.testing.assert_array_equal(oracle.linear_epilogue(Y, b, 0), Y + b[None, :])
    np.testing.assert_array_equal(oracle.linear_epilogue(Y, None, 0), Y)
    np.testing.assert_allclose(oracle.linear_epilogue(Y, b, 1),
                               torch.nn.functional.gelu(torch.from_numpy(Y + b[None, :]), approximate="tanh").numpy(),
                               rtol=1e-14)


# ---- block sizes other than 16 (NVFP4-DiT page, Algorithm 1 / Eq. 9: b in {1, 2, ..., 64}) ----------

def brute_quantize_bs(x32, S, b):
    """The brute-force quantizer with b values per scale byte (independent of the oracle)."""
    M, K = x32.shape
    packed = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // b), np.uint8)
    for i in range(M):
        for j in range(K // b):
            blk = [float(v) for v in x32[i, b * j:b * j + b]]
            byte = brute_scale_byte(max(abs(v) for v in blk), S)
            scales[i, j] = byte
            for t, v in enumerate(blk):
                k = b * j + t
                packed[i, k // 2] |= brute_code(v, byte, S) << (4 * (k & 1))
    return packed, scales


@pytest.mark.parametrize("b", [1, 2, 4, 8, 32, 64])
def test_block_size_quantizer_brute_force(b):
    """Every block size of the page's set against the exact-rational brute force (dynamic S, a zero
    block, and a static S small enough to saturate)."""
    rng = np.random.default_rng(100 + b)
    for trial in range(4):
        M, K = int(rng.integers(1, 3)), 64 * int(rng.integers(1, 3))
        x = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial == 1:
            x[:, :b] = 0.0
        S = oracle.tensor_scale(x) if trial != 2 else np.float32(oracle.tensor_scale(x) / 64)
        p, s, _ = oracle.quantize(x, S=S, block=b)
        bp, bs = brute_quantize_bs(x, float(S), b)
        np.testing.assert_array_equal(s, bs)
        np.testing.assert_array_equal(p, bp)


@pytest.mark.parametrize("b", [32, 64])
def test_block_size_equal_subblock_maxima_reduce_to_b16(b):
    """Closed form: when every 16-value sub-block of a b-block holds the b-block's maximum magnitude,
    the b-block's scale byte is each sub-block's byte and the codes are the b = 16 codes."""
    rng = np.random.default_rng(b)
    M, K = 8, 4 * b
    x = rng.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    for i in range(M):
        for j in range(K // b):
            peak = np.float32(rng.uniform(1.0, 4.0))  # above every other |value| (< 1)
            for q in range(b // 16):
                x[i, b * j + 16 * q + int(rng.integers(0, 16))] = peak if q % 2 == 0 else -peak
    S = oracle.tensor_scale(x)
    p16, s16, _ = oracle.quantize(x, S=S, block=16)
    pb, sb, _ = oracle.quantize(x, S=S, block=b)
    np.testing.assert_array_equal(pb, p16)
    np.testing.assert_array_equal(np.repeat(sb, b // 16, axis=1), s16)


@pytest.mark.parametrize("b", [2, 32, 64])
def test_block_size_dequantize_exact(b):
    """Dequantize with b values per byte: each value is RN32(q e S) of its own block's byte, checked
    against exact rationals."""
    rng = np.random.default_rng(7 * b)
    M, K = 3, 128
    packed = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (M, K // b), dtype=np.uint8)
    S = np.float32(0.0123)
    y32, _ = oracle.dequantize(packed, scales, S)
    for i in range(M):
        for k in range(K):
            code = (int(packed[i, k // 2]) >> (4 * (k & 1))) & 15
            q = Fraction(E2M1_STATED[code & 7]) * (-1 if code & 8 else 1)
            exact = q * Fraction(E4M3_TORCH[int(scales[i, k // b])]) * Fraction(float(S))
            assert y32[i, k] == np.float32(float(exact)) or (exact == 0 and y32[i, k] == 0)
