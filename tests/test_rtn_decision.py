"""The quantize kernels' division-free code decision, modelled in numpy float32.

The kernels round w / s half to even (float16 w and s) from a reciprocal r of s
(the hardware reciprocal, within one ulp of 1 / s) and t = fl(w * r): where t lies
within 2^-14 of h = floor(t) + 1/2 the code is rint(h), else rint(t). These tests
check that this decision equals the rounding of the IEEE float32 quotient that the
pages' formula q = round(w / scale) is taken as ("LLM 后训练量化深度实战…",
www.ybb.press, section 二), for every finite float16 w against a spread of float16
scales, every exact tie, and the range limit |w / s| < 341, in both evaluation
orders of t - h (rounded product, or fused multiply-add) and with r the correctly
rounded 1 / s or either float32 neighbour of it.
"""

from fractions import Fraction

import numpy as np
import pytest

BAND = np.float32(2.0 ** -14)


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _scales(n_random=160, seed=5):
    rng = np.random.default_rng(seed)
    pos = _all_finite_fp16()
    pos = pos[pos > 0]
    picks = rng.choice(pos, size=n_random, replace=False)
    special = np.array([2.0 ** -24, 3 * 2.0 ** -24, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -24, 1.0, 3.0, 7.0,
                        0.02 / 7, 1 / 7, 2047 / 1024, 65504.0, 1e-3, 5e-5], dtype=np.float16)
    return np.unique(np.concatenate([picks, special]))


ULPS = [0, -1, 1]  # r = fl(1 / s) moved by this many float32 steps (one-ulp reciprocal)


def _recip(s32, ulp):
    r = np.float32(1.0) / s32
    for _ in range(abs(ulp)):
        r = np.nextafter(r, np.float32(np.inf) if ulp > 0 else np.float32(0))
    return np.float32(r)


def _model(w32, s32, fused, ulp=0):
    """The kernels' arithmetic in float32 (fused: t - h from the exact product w * r)."""
    r = _recip(s32, ulp)
    t = w32 * r
    h = np.floor(t) + np.float32(0.5)
    if fused:
        d = (w32.astype(np.float64) * np.float64(r) - h.astype(np.float64)).astype(np.float32)
    else:
        d = t - h
    return np.rint(np.where(np.abs(d) < BAND, h, t))


@pytest.mark.parametrize("ulp", ULPS)
@pytest.mark.parametrize("fused", [False, True])
def test_decision_equals_ieee_quotient_all_fp16(fused, ulp):
    w = _all_finite_fp16().astype(np.float32)
    for s16 in _scales():
        s32 = np.float32(s16)
        ref = np.rint(w / s32)
        got = _model(w, s32, fused, ulp)
        inside = np.abs(ref) < 340
        bad = inside & (got != ref)
        assert not bad.any(), (float(s16), ulp, w[bad][:4])
        # past the range the decision may differ by one but stays beyond every clamp bound
        assert np.all(np.abs(got[~inside]) >= 339)


@pytest.mark.parametrize("ulp", ULPS)
@pytest.mark.parametrize("fused", [False, True])
def test_exact_ties_round_to_even(fused, ulp):
    checked = 0
    for s16 in _scales():
        s = Fraction(float(s16))
        for k in range(-130, 130):
            w_exact = (Fraction(2 * k + 1, 2)) * s
            with np.errstate(over="ignore"):  # past the float16 range: skipped below
                w16 = np.float16(float(w_exact))
            if not np.isfinite(w16) or Fraction(float(w16)) != w_exact:
                continue  # not a float16 value
            got = _model(np.array([w16], dtype=np.float32), np.float32(s16), fused, ulp)[0]
            even = k if k % 2 == 0 else k + 1
            assert got == even, (float(s16), float(w16))
            checked += 1
    assert checked > 1000


def test_non_ties_keep_the_gap():
    # the margin the decision relies on: a quotient that is not a half-integer
    # stays at least 2^-12 away from every half-integer (1/(2 m_s) >= 1/4094 when
    # w's exponent reaches s's minus 1; 1/2 - 2^-12 at most below that)
    w = _all_finite_fp16().astype(np.float64)
    w = w[(w > 0) & (w < 2048)]
    for s16 in _scales(40, seed=9):
        q = w / float(s16)
        q = q[q < 600]
        dist = np.abs(q - (np.floor(q) + 0.5))
        assert np.all((dist == 0) | (dist >= 2.0 ** -12)), float(s16)


def test_zero_scale_gives_code_zero():
    # the kernels use r = 0 for s == 0: every weight gets q = 0
    w = _all_finite_fp16().astype(np.float32)
    t = w * np.float32(0.0)
    h = np.floor(t) + np.float32(0.5)
    assert np.all(np.rint(np.where(np.abs(t - h) < BAND, h, t)) == 0)


@pytest.mark.parametrize("d", [7, 127])
def test_scale_from_reciprocal_constant(d):
    # the INT4 (amax / 7), KV (amax / 7) and INT8 (amax / 127) scales are formed as
    # fp16(amax * fl(1 / d)) instead of fp16(fl(amax / d)): equal for every positive
    # float16 amax (the float32 multiply is correctly rounded, so this model is exact)
    a = _all_finite_fp16()
    a = a[a > 0].astype(np.float32)
    c = np.float32(1.0) / np.float32(d)
    ref = (np.maximum(a, np.float32(1e-12)) / np.float32(d)).astype(np.float16)
    got = (np.maximum(a, np.float32(1e-12)) * c).astype(np.float16)
    assert np.array_equal(ref.view(np.uint16), got.view(np.uint16))
