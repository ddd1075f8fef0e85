"""Property tests of the oracle (CPU): Hypothesis draws 16-value blocks and tensor scales, including
the adversarial cases of the format, and every draw is checked against exact-rational brute force
and the invariants [NVFP4-DiT page, Methodology section 1, Definition III.1 (round to the E2M1
grid, clip to +-6, block scale) and Lemma III.2 (error bound, in the half-ulp reading); vllm-omni
NVFP4 RFC, Motivation (E4M3 block scale under an fp32 tensor scale)].

Block kinds: plain random values over many binades; exact ties, i.e. a block whose amax lands on
6 e S for an E4M3 value e and whose other values sit on the decision boundaries t e S; blocks whose
ratio amax / (6 S) lies on an E4M3 midpoint; tiny blocks (subnormal E4M3 scales, flushed blocks);
blocks far above 448 * 6 * S (saturated scale, clipped codes); signed zeros everywhere.  Draws
are derandomized, so the suite is reproducible.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from test_oracle_pins import brute_quantize

E4M3_VALUES = [float(v) for v in torch.arange(1, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float()]
BOUNDARIES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

scales = st.one_of(
    st.sampled_from([2.0 ** -8, 2.0 ** -9, 1.0, 1.1 * 2.0 ** -9, 1.5 * 2.0 ** -9, 2.0 ** -8 / 3, 1.0 / 2688,
                     1.75 * 2.0 ** -10, 2.0 ** -30, 3.0 * 2.0 ** 10]),
    st.floats(min_value=2.0 ** -40, max_value=2.0 ** 20, width=32, allow_subnormal=False))


def f32(v: float) -> float:
    return float(np.float32(v))


@st.composite
def block(draw, S):
    kind = draw(st.sampled_from(["random", "ties", "midpoint", "tiny", "huge"]))
    signs = draw(st.lists(st.booleans(), min_size=16, max_size=16))
    if kind == "random":
        k = draw(st.integers(min_value=-20, max_value=12))
        mags = draw(st.lists(st.floats(min_value=0.0, max_value=2.0, width=32), min_size=16, max_size=16))
        vals = [f32(m * 2.0 ** k) for m in mags]
    elif kind == "ties":
        e = draw(st.sampled_from(E4M3_VALUES))
        ts = draw(st.lists(st.sampled_from(BOUNDARIES + GRID), min_size=15, max_size=15))
        vals = [f32(6.0 * e * S)] + [f32(t * e * S) for t in ts]
    elif kind == "midpoint":
        i = draw(st.integers(min_value=0, max_value=len(E4M3_VALUES) - 2))
        mid = 0.5 * (E4M3_VALUES[i] + E4M3_VALUES[i + 1])
        rest = draw(st.lists(st.floats(min_value=0.0, max_value=1.0, width=32), min_size=15, max_size=15))
        amax = f32(6.0 * mid * S)
        vals = [amax] + [f32(r * amax) for r in rest]
    elif kind == "tiny":
        j = draw(st.integers(min_value=8, max_value=14))
        mags = draw(st.lists(st.floats(min_value=0.0, max_value=6.0, width=32), min_size=16, max_size=16))
        vals = [f32(m * S * 2.0 ** -j) for m in mags]
    else:
        k = draw(st.integers(min_value=12, max_value=30))
        mags = draw(st.lists(st.floats(min_value=0.0, max_value=1.0, width=32), min_size=16, max_size=16))
        vals = [f32(m * 6 * 448 * S * 2.0 ** k) for m in mags]
    zeros = draw(st.lists(st.booleans(), min_size=16, max_size=16))
    out = [0.0 if z and draw(st.booleans()) else v for v, z in zip(vals, zeros)]
    return [-v if s else v for v, s in zip(out, signs)]


@st.composite
def static_case(draw):
    S = f32(draw(scales))
    nblk = draw(st.integers(min_value=1, max_value=3))
    x = np.array([draw(block(S)) for _ in range(nblk)], np.float32).reshape(1, -1)
    return x, S


def _finite(x):
    return np.isfinite(x).all()


@SETTINGS
@given(static_case())
def test_oracle_equals_brute_force_static(case):
    """The C oracle and the exact-rational brute force agree on every byte, under a static S."""
    x, S = case
    if not _finite(x):
        return
    p, s, _ = oracle.quantize(x, S=S)
    bp, bs = brute_quantize(x, S)
    assert np.array_equal(s, bs)
    assert np.array_equal(p, bp)


@SETTINGS
@given(static_case())
def test_oracle_equals_brute_force_dynamic(case):
    """The same with the dynamic tensor scale S = RN32(amax / 2688)."""
    x, _ = case
    if not _finite(x) or np.max(np.abs(x)) < 2.0 ** -100:  # S would be subnormal: outside the contract
        return
    p, s, S = oracle.quantize(x)
    assert np.float32(S) == np.float32(np.float32(np.max(np.abs(x))) / np.float32(2688.0))
    bp, bs = brute_quantize(x, float(S))
    assert np.array_equal(s, bs) and np.array_equal(p, bp)


@SETTINGS
@given(static_case())
def test_invariants(case):
    """|q| <= 6, signs copied (also of zeros), monotone codes within a block, zero blocks get byte
    0, bytes <= 0x7E, a scale byte >= 3 puts the block maximum on code 6, and for in-range values
    the error is at most half an E2M1 ulp of v's binade: |Q(v) - v| <= 2^-3 2^(floor(log2 x) + 1) e S
    with x = |v| / (e S) in [1, 6]."""
    x, S = case
    if not _finite(x):
        return
    p, s, _ = oracle.quantize(x, S=S)
    y, _ = oracle.dequantize(p, s, S)
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(x.shape)
    assert (s <= 0x7E).all()
    assert ((codes >> 3).astype(bool) == np.signbit(x)).all()
    xb, cb, yb = x.reshape(-1, 16).astype(np.float64), (codes & 7).reshape(-1, 16), y.reshape(-1, 16)
    for j in range(xb.shape[0]):
        e = E4M3_VALUES[s[0, j] - 1] if s[0, j] else 0.0
        a = np.abs(xb[j])
        if a.max() == 0:
            assert s[0, j] == 0
        if s[0, j] >= 3:
            assert cb[j].max() == 7
        order = np.argsort(a, kind="stable")
        assert (np.diff(cb[j][order]) >= 0).all()
        assert (np.abs(yb[j]) <= 6 * e * S * (1 + 2.0 ** -22)).all()
        if e == 0:
            continue
        xs = a / (e * S)
        inr = (xs >= 1.0) & (xs <= 6.0)
        bound = 2.0 ** -3 * 2.0 ** (np.floor(np.log2(np.where(inr, xs, 1.0))) + 1) * e * S
        err = np.abs(yb[j].astype(np.float64) - xb[j])
        # y is RN32 of the exact Q(v): allow its rounding
        assert (err[inr] <= bound[inr] + np.abs(yb[j][inr]) * 2.0 ** -24).all()


@SETTINGS
@given(static_case())
def test_requantize_idempotent(case):
    """Requantizing the fp32 dequantization with the same static S reproduces every byte of each
    block whose scale byte is 0x00 or >= 0x03 (the reading of the idempotence claim)."""
    x, S = case
    if not _finite(x):
        return
    p, s, _ = oracle.quantize(x, S=S)
    y, _ = oracle.dequantize(p, s, S)
    p2, s2, _ = oracle.quantize(y, S=S)
    keep = (s[0] == 0) | (s[0] >= 3)
    assert np.array_equal(s2[0][keep], s[0][keep])
    pb, p2b = p.reshape(-1, 8), p2.reshape(-1, 8)
    assert np.array_equal(p2b[keep], pb[keep])


@SETTINGS
@given(static_case(), st.sampled_from([32, 64]))
def test_block_sizes_equal_subblock_maxima(case, b):
    """A b-block made of one 16-block repeated b / 16 times has that 16-block's maximum, so block
    size b gives the b = 16 bytes (each scale byte once per b-block)."""
    x, S = case
    if not _finite(x):
        return
    reps = b // 16
    xb = np.concatenate([np.tile(blk, reps) for blk in x.reshape(-1, 16)]).astype(np.float32).reshape(1, -1)
    p16, s16, _ = oracle.quantize(xb, S=S)
    pb, sb, _ = oracle.quantize(xb, S=S, block=b)
    assert np.array_equal(pb, p16)
    assert np.array_equal(sb[0], s16[0][::reps])
