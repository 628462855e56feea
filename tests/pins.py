"""Checks that pin the oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a value a page prints, a closed form, an exhaustive enumeration or an exact
brute force. ``tests/test_oracle_pins.py`` runs every pin on the oracle as it
is; ``tests/test_oracle_mutations.py`` plants plausible mistakes into the
oracle (on the CPU) and checks that at least one pin catches each of them.

The functions look up the oracle through ``import oracle`` at call time so a
monkeypatched oracle is what they test.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import exact_round as xr  # noqa: E402
import synth  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _orc():
    import oracle

    return oracle


# ---------------------------------------------------------------- page values


def pin_scalar_rounding_example():
    """3.14159 at scale 0.01 -> code 314, dequant 3.14, error 0.00159 (page iopencloud, 1.2)."""
    o = _orc()
    gd = _golden("iopencloud_rounding_example.json")
    q, w_hat, err = o.rtn_scalar(gd["w"], gd["scale"])
    assert q == gd["printed"]["q"], q
    assert abs(w_hat - gd["printed"]["dequant"]) < 1e-12
    assert abs(err - gd["printed"]["abs_error"]) < 5e-9
    # Under INT4 bounds the same input clamps to the top code.
    q4, w4, _ = o.rtn_scalar(gd["w"], gd["scale"], -8, 7)
    assert q4 == 7 and abs(w4 - 0.07) < 1e-12


def pin_awq_rtn_table():
    """Four-weight row of the RTN/AWQ table (page arganzheng, 六.2)."""
    o = _orc()
    gd = _golden("arg_awq_rtn_table.json")
    x = np.array(gd["x"])
    w = np.array(gd["chosen"]["w"])
    pr = gd["printed"]
    assert abs(float(x @ w) - pr["Y_unquantized"]) < 5e-4
    for key in ("rtn", "awq"):
        cs = np.array(pr[key]["channel_scale"], dtype=np.float64)
        q, s = o.quantize_sym_exact((w * cs)[None, :], gd["group_size"])
        assert list(q[0]) == pr[key]["codes"], (key, q)
        w_hat = o.dequant_sym(q, s, gd["group_size"])[0]
        assert np.allclose(w_hat, pr[key]["dequant"], atol=5e-5), (key, w_hat)
        x_used = x / cs
        assert np.allclose(x_used, pr[key]["x_used"])
        y_hat = float(o.gemm_ref(x_used[None, :], w_hat[None, :])[0, 0])
        assert abs(y_hat - pr[key]["y_hat"]) < 5e-5, (key, y_hat)
        assert abs((y_hat - pr["Y_unquantized"]) - pr[key]["y_err"]) < 2e-4
    # relative error of the second weight before/after the channel scaling
    q, s = o.quantize_sym_exact(w[None, :], 4)
    rel = abs(o.dequant_sym(q, s, 4)[0, 1] - w[1]) / w[1]
    assert abs(rel - pr["col2_relative_error_rtn"]) < 5e-4
    q, s = o.quantize_sym_exact((w * [1, 2.5, 1, 1])[None, :], 4)
    rel = abs(o.dequant_sym(q, s, 4)[0, 1] / 2.5 - w[1]) / w[1]
    assert abs(rel - pr["col2_relative_error_awq"]) < 5e-4


def pin_awq_table_fp16_storage():
    """The same row through the float16 path: codes unchanged, y_hat within 5e-4."""
    o = _orc()
    gd = _golden("arg_awq_rtn_table.json")
    w16 = np.array(gd["chosen"]["w"], dtype=np.float16)[None, :]
    q, s16 = o.quantize_sym(w16, 4)
    assert list(q[0]) == gd["printed"]["rtn"]["codes"]
    y = o.gemm_ref(np.array(gd["x"], dtype=np.float16)[None, :], o.dequant_sym(q, s16, 4))[0, 0]
    assert abs(y - gd["printed"]["rtn"]["y_hat"]) < 5e-4


def pin_rotation_scale_ratio():
    """amax / scale = 7 for both printed (amax, scale) pairs (page arganzheng, 八.2)."""
    o = _orc()
    pr = _golden("arg_rotation_scale.json")["printed"]
    for a, s in ((pr["amax"], pr["int4_scale"]), (pr["amax_rotated"], pr["int4_scale_rotated"])):
        s_or = float(o.sym_scale_fp16(np.array([a], dtype=np.float16))[0])
        # printed values have 3-4 significant digits; fp16 storage adds 2^-11
        assert abs(s_or - s) / s < 2e-3, (a, s, s_or)
        _, s_exact = o.quantize_sym_exact(np.array([[a, 0.0]]), 2)
        assert abs(float(s_exact[0, 0]) - s) / s < 1.5e-3


# ---------------------------------------------------------------- invariants


def pin_sym_invariants(N=64, K=1024, g=128, seed=11):
    """Group max -> +-7, |w - w_hat| <= s16/2, no code -8 (page ybb 二; page arganzheng 三.1)."""
    o = _orc()
    W = synth.weight(N, K, seed=seed)
    q, s16 = o.quantize_sym(W, g)
    assert q.dtype == np.int8 and q.shape == (N, K) and s16.shape == (N, K // g)
    assert q.min() >= -7 and q.max() <= 7, "code -8 must never occur"
    Wg = W.reshape(N, K // g, g).astype(np.float64)
    qg = q.reshape(N, K // g, g)
    idx = np.abs(Wg).argmax(axis=2)
    at_max = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    sign = np.sign(np.take_along_axis(Wg, idx[..., None], axis=2)[..., 0])
    assert np.all(at_max == 7 * sign)
    w_hat = o.dequant_sym(q, s16, g)
    bound = np.repeat(s16.astype(np.float64), g, axis=1) / 2
    assert np.all(np.abs(W.astype(np.float64) - w_hat) <= bound)


def pin_exact_grid_recovered(seed=3):
    """Weights already on the grid k*2^-6 with |k| <= 7 and a +-7 per group come back unchanged."""
    o = _orc()
    r = np.random.default_rng(seed)
    N, K, g = 8, 256, 32
    k = r.integers(-7, 8, size=(N, K))
    k.reshape(N, K // g, g)[:, :, 5] = np.where(r.random((N, K // g)) < 0.5, -7, 7)
    W = (k * 2.0 ** -6).astype(np.float16)
    q, s16 = o.quantize_sym(W, g)
    assert np.all(s16 == np.float16(2.0 ** -6))
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(o.dequant_sym(q, s16, g), W.astype(np.float64))


def pin_ties_half_even():
    """Exact half-integer quotients round to even (the pages' torch.round)."""
    o = _orc()
    # amax 1.75 -> s16 = 0.25; 0.625/0.25 = 2.5 -> 2, 0.375/0.25 = 1.5 -> 2, -0.625 -> -2, 0.125 -> 0
    W = np.array([[1.75, 0.625, 0.375, -0.625, 0.125, -0.125, 0.875, -1.125]], dtype=np.float16)
    q, s16 = o.quantize_sym(W, 8)
    assert float(s16[0, 0]) == 0.25
    assert list(q[0]) == [7, 2, 2, -2, 0, 0, 4, -4]


def pin_zero_group():
    """All-zero group: scale 0 and codes 0 (reading R4); other groups unaffected."""
    o = _orc()
    W = np.zeros((2, 64), dtype=np.float16)
    W[1, 32:] = np.float16(0.5)
    W[0, 40] = np.float16(-0.7)
    q, s16 = o.quantize_sym(W, 32)
    assert s16[0, 0] == 0 and s16[1, 0] == 0 and np.all(q[:, :32] == 0)
    assert q[0, 40] == -7 and np.all(q[1, 32:] == 7)


def pin_scale_exhaustive():
    """fp16(fp32(a)/7) is the correctly rounded a/7 for every positive finite float16 a."""
    o = _orc()
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    a = bits.view(np.float16)
    s = o.sym_scale_fp16(a)
    cand = (a.astype(np.float64) / 7.0).astype(np.float16)
    # The float64 quotient can only mis-round into float16 if a/7 sat within
    # 2^-53 (relative) of a float16 rounding midpoint; a/7 with an 11-bit a is
    # at least 2^-14/7 away from any midpoint it does not equal, and a/7 equals
    # a midpoint only if 7 divides the integer a * 2^-e. Check those exactly.
    assert np.array_equal(s.view(np.uint16), cand.view(np.uint16))
    for ai, si in zip(a[::97], s[::97]):
        v = Fraction(float(ai)) / 7
        lo = np.nextafter(si, np.float16(0))
        hi = np.nextafter(si, np.float16(np.inf))
        d = abs(v - Fraction(float(si)))
        assert d <= abs(v - Fraction(float(lo))) and d <= abs(v - Fraction(float(hi)))


def pin_code_decision_exact(n_scales=120, seed=5):
    """rint of the IEEE float32 quotient equals rint of the exact rational w/s16.

    For each sampled scale, every float16 w with |w| <= 7.5*s16 is tested. The
    float64 quotient decides the rounding exactly (its error is below 2^-49 while
    a non-tie quotient of two float16 numbers is at least 2^-12 from a
    half-integer); quotients within 1e-9 of a half-integer are re-checked with
    Fractions.
    """
    o = _orc()
    r = np.random.default_rng(seed)
    sb = np.concatenate([r.integers(0x0400, 0x5000, size=n_scales - 4), [0x0001, 0x0100, 0x1C00, 0x3C00]])
    all16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    all16 = np.concatenate([all16, -all16[1:]])
    for b in sb.astype(np.uint16):
        s16 = np.array([b], dtype=np.uint16).view(np.float16)
        sv = float(s16[0])
        # group of the candidates plus one element at 7*s16 so the group scale is s16
        amax = np.float16(7 * sv)
        if o.sym_scale_fp16(np.array([amax]))[0] != s16[0]:
            continue
        w = all16[np.abs(all16.astype(np.float64)) <= float(amax)]
        if w.size < 2:
            continue
        q32 = np.clip(np.rint(w.astype(np.float32) / np.float32(sv)), -8, 7)
        q64 = np.clip(np.rint(w.astype(np.float64) / sv), -8, 7)
        assert np.array_equal(q32, q64), sv
        near = np.abs(np.abs(w.astype(np.float64) / sv) % 1.0 - 0.5) < 1e-9
        for wi, qi in zip(w[near], q64[near]):
            fq = Fraction(float(wi)) / Fraction(sv)
            fl = fq.numerator // fq.denominator
            frac = fq - fl
            exact = fl if frac < Fraction(1, 2) else fl + 1 if frac > Fraction(1, 2) else (fl if fl % 2 == 0 else fl + 1)
            assert qi == max(-8, min(7, exact))
        # and the oracle itself: a row [amax, w...] padded to the group size
        g = 32
        n_full = (w.size // (g - 1)) * (g - 1)
        if n_full == 0:
            continue
        rows = w[:n_full].reshape(-1, g - 1)
        Wm = np.concatenate([np.full((rows.shape[0], 1), amax, dtype=np.float16), rows], axis=1)
        q, s_or = o.quantize_sym(Wm, g)
        assert np.all(s_or == s16[0])
        assert np.array_equal(q[:, 1:].astype(np.float64).ravel(), q64[:n_full])


def pin_noise_model(N=1024, K=4096, seed=0, groups=(4096, 512, 128, 32)):
    """MSE matches the uniform-noise model E[e^2] = Delta^2/12 (page arganzheng, 三.1).

    Refinement: the group's largest element is reproduced exactly, so the model
    is mean over groups of ((g-1)/g) * s16^2/12. Also checks the ordering of the
    page ybb's section 二 demo: MSE falls as the group shrinks.
    """
    o = _orc()
    W = synth.weight(N, K, seed=seed)
    mse_of = {}
    for g in groups:
        q, s16 = o.quantize_sym(W, g)
        mse = o.quant_mse(W, o.dequant_sym(q, s16, g))
        model = float(np.mean(s16.astype(np.float64) ** 2)) / 12 * (g - 1) / g
        assert abs(mse / model - 1) < 0.005, (g, mse, model)
        mse_of[g] = mse
    # the ordering the page prints (its magnitudes are not reproducible; the model above fixes them)
    printed = {int(k): v for k, v in _golden("ybb_mse_by_group.json")["printed_mse"].items()}
    by_printed = sorted(printed, key=lambda g: -printed[g])
    assert [g for g in sorted(mse_of, key=lambda g: -mse_of[g]) if g in printed] == by_printed, mse_of


def pin_asym_exact_grid(seed=7):
    """A group already on the uint4 grid (min -> code 0, max -> code 15) comes back unchanged."""
    o = _orc()
    r = np.random.default_rng(seed)
    N, K, g = 6, 128, 32
    z_true = r.integers(1, 15, size=(N, K // g))
    q_true = r.integers(0, 16, size=(N, K))
    qg = q_true.reshape(N, K // g, g)
    qg[:, :, 0] = 0
    qg[:, :, 1] = 15
    W = ((q_true - np.repeat(z_true, g, axis=1)) * 2.0 ** -5).astype(np.float16)
    q, s16, z = o.quantize_asym(W, g)
    assert np.all(s16 == np.float16(2.0 ** -5))
    assert np.array_equal(z.astype(np.int64), z_true)
    assert np.array_equal(q.astype(np.int64), q_true)
    assert np.array_equal(o.dequant_asym(q, s16, z, g), W.astype(np.float64))


def _asym_pairs(n=100_000, seed=61):
    """float16 (min, max) pairs: straddling zero, one-sided on either side, equal,
    and hand-picked ones whose float32 range is not a float16 value (so rounding
    the range to float16 first would move the scale) or exceeds the float16 range."""
    r = np.random.default_rng(seed)
    neg = r.integers(0x8000, 0xFBFF, size=n, endpoint=True).astype(np.uint16).view(np.float16)
    pos = r.integers(0x0000, 0x7BFF, size=n, endpoint=True).astype(np.uint16).view(np.float16)
    a, b = neg.copy(), pos.copy()
    k = n // 7
    a[:k], b[:k] = pos[:k], pos[k:2 * k]                   # both >= 0: z clamps to 0
    a[k:2 * k], b[k:2 * k] = neg[:k], neg[k:2 * k]         # both <= 0: z clamps to 15
    mn, mx = np.minimum(a, b), np.maximum(a, b)
    hand = [(-2.0 ** -14, 1.0), (-0.3, 1000.7), (-65504.0, 65504.0), (-60000.0, 30000.0), (0.0, 0.0),
            (1.5, 1.5), (-2.0 ** -24, 2.0 ** -24), (-1.0, 2.0 ** -13), (-3.0, 5.0), (-7.5, 7.5)]
    hm = np.array([h[0] for h in hand], dtype=np.float16)
    hx = np.array([h[1] for h in hand], dtype=np.float16)
    return np.concatenate([hm, mn]), np.concatenate([hx, mx])


def pin_asym_scale_zero_exact(g=8, seed=62):
    """Reading R5 step by step in exact integer arithmetic, on 10^5 float16 (min, max)
    pairs: range = fl32(fl32(max) - fl32(min)), s16 = fp16(fl32(range / 15)),
    z = clamp(rint(-min / s16), 0, 15), q = clamp(rint(w / s16) + z, 0, 15) with
    rint half to even of the exact rational quotient, q = z = 0 where s16 == 0
    ([ARG] section 二.2; [WIKI] section 7.4.1.1). Each group holds its min, its max
    and g - 2 values drawn between them."""
    o = _orc()
    mn, mx = _asym_pairs()
    G = mn.size
    r = np.random.default_rng(seed)
    lo, hi = mn.astype(np.float64)[:, None], mx.astype(np.float64)[:, None]
    mid = (lo + (hi - lo) * r.random((G, g - 2))).astype(np.float16)
    W = np.concatenate([mn[:, None], mid, mx[:, None]], axis=1)
    W = np.take_along_axis(W, r.permuted(np.tile(np.arange(g), (G, 1)), axis=1), axis=1)
    q, s16, z = o.quantize_asym(W, g)
    # the range: an exact integer on the 2^-24 grid, rounded once to float32
    D = xr.on_grid(mx) - xr.on_grid(mn)
    Qr, Tr = xr.round_to(D, -24, False, xr.FP32)
    # / 15 rounded to float32, then to float16
    Qd, Td, st = xr.divide(Qr, Tr, 15)
    Q32, T32 = xr.round_to(Qd, Td, st, xr.FP32)
    Q16, T16 = xr.round_to(Q32, T32, False, xr.FP16)
    s_exp = xr.to_float64(Q16, T16)
    got = s16[:, 0].astype(np.float64)
    assert np.array_equal(got, s_exp), np.flatnonzero(got != s_exp)[:5]
    # z and q from exact integer quotients: w / s16 = (w * 2^24) / (Q16 * 2^(T16 + 24))
    S = np.where(Q16 > 0, Q16 << np.maximum(T16 + 24, 0), 1)
    zero = Q16 == 0
    z_exp = np.where(zero, 0, np.clip(xr.rint_div(-xr.on_grid(mn), S), 0, 15))
    assert np.array_equal(z[:, 0].astype(np.int64), z_exp)
    Wi = xr.on_grid(W)
    q_exp = np.clip(xr.rint_div(Wi, S[:, None]) + z_exp[:, None], 0, 15)
    q_exp = np.where(zero[:, None], 0, q_exp)
    assert np.array_equal(q.astype(np.int64), q_exp)


def pin_asym_invariants(N=64, K=1024, g=64, seed=9):
    """Asymmetric bounds: codes in [0,15], the group min maps to code 0 when z is
    unclamped, |w - w_hat| <= s16/2 below the clamp and <= 1.5*s16 at it."""
    o = _orc()
    W, _ = synth.heavy_tailed_weight(N, K, seed=seed)
    q, s16, z = o.quantize_asym(W, g)
    assert q.max() <= 15 and z.max() <= 15
    Wg = W.reshape(N, K // g, g).astype(np.float64)
    qg = q.reshape(N, K // g, g).astype(np.int64)
    imin = Wg.argmin(axis=2)
    qmin = np.take_along_axis(qg, imin[..., None], axis=2)[..., 0]
    unclamped = (z > 0) & (z < 15)
    assert np.all(qmin[unclamped] == 0)
    w_hat = o.dequant_asym(q, s16, z, g)
    err = np.abs(W.astype(np.float64) - w_hat)
    s_rep = np.repeat(s16.astype(np.float64), g, axis=1)
    zin = np.repeat(unclamped, g, axis=1)
    inner = (q > 0) & (q < 15) & zin
    assert np.all(err[inner] <= s_rep[inner] / 2)
    assert np.all(err[zin] <= 1.5 * s_rep[zin] * (1 + 2 ** -10))


def pin_asym_noise_model(N=512, K=4096, seed=1):
    """Asymmetric MSE ~ Delta^2/12 with Delta = (max-min)/15 (page arganzheng, 三.1)."""
    o = _orc()
    W = synth.weight(N, K, seed=seed)
    for g in (128, 32):
        q, s16, z = o.quantize_asym(W, g)
        mse = o.quant_mse(W, o.dequant_asym(q, s16, z, g))
        model = float(np.mean(s16.astype(np.float64) ** 2)) / 12
        assert abs(mse / model - 1) < 0.02, (g, mse, model)


# ---------------------------------------------------------------- packing / layout


def pin_canonical_hand_bytes():
    o = _orc()
    q = np.array([[-8, -7, -6, -5, -4, -3, -2, -1], [0, 1, 2, 3, 4, 5, 6, 7]])
    b = o.pack_canonical(q)
    assert list(b[0]) == [0x98, 0xBA, 0xDC, 0xFE]
    assert list(b[1]) == [0x10, 0x32, 0x54, 0x76]
    assert np.array_equal(o.unpack_canonical(b), q)
    assert list(o.unpack_canonical(np.array([[0x10, 0xF1]], dtype=np.uint8), signed=False)[0]) == [0, 1, 1, 15]


def pin_device_layout_hand_positions():
    """Single codes planted at hand-computed positions of the device layout spec."""
    o = _orc()
    N, K = 40, 352                       # 3 row tiles (last ragged), 3 super-blocks (last ragged)
    sh = o.device_shapes(N, K, 32)
    assert (sh["Np"], sh["Kp"], sh["S"], sh["Gp"], sh["code_bytes"]) == (48, 384, 3, 12, 48 * 384 // 2)
    # (n, k, expected byte, expected nibble): worked by hand from the spec
    #   n=17,k=200: t=1 r=1 s=1 m=2 c=1 e=0 -> lane 17, p=0 -> ((1*3+1)*64+17)*16+8+0 = 4376, low
    #   n=0,k=1:    t=0 r=0 s=0 m=0 c=0 e=1 -> lane 0,  p=4 -> 2, low
    #   n=15,k=127: t=0 r=15 s=0 m=3 c=3 e=7 -> lane 63, p=7 -> 63*16+12+3 = 1023, high
    #   n=39,k=350: t=2 r=7 s=2 m=2 c=3 e=6 -> lane 55, p=3 -> ((2*3+2)*64+55)*16+8+1 = 9081, high
    cases = [(17, 200, 4376, 0), (0, 1, 2, 0), (15, 127, 1023, 4), (39, 350, 9081, 4)]
    for n, k, byte, shift in cases:
        q = np.zeros((N, K), dtype=np.int64)
        q[n, k] = 5
        dev = o.codes_to_device(q, symmetric=True)
        # every other nibble holds 8 (code 0 in offset binary)
        expect_byte = (0x88 & ~(0xF << shift)) | (13 << shift)
        assert dev[byte] == expect_byte, (n, k, hex(dev[byte]))
        others = np.delete(dev, byte)
        assert np.all(others == 0x88)
        back = o.codes_from_device(dev, N, K)
        assert np.array_equal(back, q.astype(np.int8))
        q_a = np.zeros((N, K), dtype=np.int64)
        q_a[n, k] = 11
        dev_a = o.codes_to_device(q_a, symmetric=False)
        assert dev_a[byte] == (11 << shift) and np.count_nonzero(dev_a) == 1


def pin_device_layout_bijection(seed=2):
    o = _orc()
    r = np.random.default_rng(seed)
    for N, K in ((16, 128), (33, 96), (5, 32), (48, 1024)):
        q = r.integers(-8, 8, size=(N, K))
        dev = o.codes_to_device(q)
        assert dev.size == o.device_shapes(N, K, 32)["code_bytes"]
        assert np.array_equal(o.codes_from_device(dev, N, K), q.astype(np.int8))
        # a permutation: the multiset of valid nibbles is preserved
        qa = r.integers(0, 16, size=(N, K))
        da = o.codes_to_device(qa, symmetric=False)
        nib = np.concatenate([da & 0xF, da >> 4]).astype(np.int64)
        assert np.array_equal(np.bincount(nib, minlength=16) - np.bincount(qa.ravel(), minlength=16),
                              np.eye(16, dtype=np.int64)[0] * (nib.size - qa.size))
    # group-wise arrays: [t, j, r] addressing
    s = np.arange(20 * 3, dtype=np.float16).reshape(20, 3)
    d = o.groupwise_to_device(s, 20, 96, 32)
    assert d.shape == (2, 4, 16)         # Kp = 128 -> Gp = 4, the last group is padding
    assert d[1, 2, 3] == s[19, 2] and d[1, 2, 4] == 0 and d[0, 1, 15] == s[15, 1]
    assert np.all(d[:, 3, :] == 0)
    assert np.array_equal(o.groupwise_from_device(d, 20, 96, 32), s)


# ---------------------------------------------------------------- product


def _exact_product(x16, q, s16, g, z=None):
    """Exact rational y = x . w_hat^T from the codes (pure-Python brute force)."""
    B, K = x16.shape
    N = q.shape[0]
    out = np.zeros((B, N))
    for b in range(B):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                zz = 0 if z is None else int(z[n, k // g])
                acc += Fraction(float(x16[b, k])) * Fraction(float(s16[n, k // g])) * (int(q[n, k]) - zz)
            out[b, n] = float(acc)
    return out


def pin_product_bruteforce(seed=4):
    o = _orc()
    for B, N, K, g in ((1, 5, 32, 32), (3, 17, 64, 32), (2, 4, 256, 64), (3, 3, 128, 128)):
        W = synth.weight(N, K, seed=seed + N)
        x = synth.activation(B, K, seed=seed + K)
        q, s16 = o.quantize_sym(W, g)
        y = o.gemm_ref(x, o.dequant_sym(q, s16, g))
        assert y.shape == (B, N)
        ye = _exact_product(x, q, s16, g)
        assert np.allclose(y, ye, rtol=1e-12, atol=1e-15)
        qa, sa, za = o.quantize_asym(W, g)
        ya = o.gemm_ref(x, o.dequant_asym(qa, sa, za, g))
        assert np.allclose(ya, _exact_product(x, qa, sa, g, za), rtol=1e-12, atol=1e-15)
        rows = [N - 1, 0]
        assert np.allclose(o.gemm_ref_rows(x, q, s16, g, rows), ye[:, rows], rtol=1e-12, atol=1e-15)


def pin_product_special_cases():
    o = _orc()
    K, g = 256, 128
    x = synth.activation(2, K, seed=1)
    # all weights 1.0: s16 = fp16(1/7), codes 7, y = 7*s16*sum(x)
    W = np.ones((3, K), dtype=np.float16)
    q, s16 = o.quantize_sym(W, g)
    y = o.gemm_ref(x, o.dequant_sym(q, s16, g))
    assert np.allclose(y, 7 * float(s16[0, 0]) * x.astype(np.float64).sum(axis=1, keepdims=True), rtol=1e-13)
    # one-hot rows pick single activations
    W = np.zeros((4, K), dtype=np.float16)
    hot = [3, 100, 130, 255]
    for i, k in enumerate(hot):
        W[i, k] = np.float16(0.5 + i)
    q, s16 = o.quantize_sym(W, g)
    y = o.gemm_ref(x, o.dequant_sym(q, s16, g))
    for i, k in enumerate(hot):
        assert np.allclose(y[:, i], 7 * float(s16[i, k // g]) * x[:, k].astype(np.float64), rtol=1e-13)
    # zero weights
    q, s16 = o.quantize_sym(np.zeros((2, K), dtype=np.float16), g)
    assert np.all(o.gemm_ref(x, o.dequant_sym(q, s16, g)) == 0)
    # linearity in x
    W = synth.weight(5, K, seed=8)
    q, s16 = o.quantize_sym(W, g)
    wh = o.dequant_sym(q, s16, g)
    x1 = synth.activation(1, K, seed=2).astype(np.float64)
    x2 = synth.activation(1, K, seed=3).astype(np.float64)
    assert np.allclose(o.gemm_ref(2 * x1 - x2, wh), 2 * o.gemm_ref(x1, wh) - o.gemm_ref(x2, wh), rtol=1e-12, atol=1e-12)


# ------------------------------------------- clipping search ([ARG] section 三.2)


def _round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def pin_clip_100_is_rtn(seed=21):
    """With only alpha = 1 to search, the clipping search is RTN bit for bit."""
    o = _orc()
    for g in (32, 64, 128, 256):
        W = synth.weight(32, 1024, seed=seed + g)
        q, s, p = o.quantize_sym_clip(W, g, 100)
        q0, s0 = o.quantize_sym(W, g)
        assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))
        assert np.all(p == 100)


def pin_clip_scale_rounding(seed=23):
    """s16_p lies within 2^-10.9 (relative) of the exact p/100 * amax / 7, grows with p,
    and equals the RTN scale at p = 100."""
    o = _orc()
    rng = np.random.default_rng(seed)
    amax = np.concatenate([rng.uniform(1e-3, 60000, 4000), 7.0 * 2.0 ** np.arange(-14, 13)]).astype(np.float16)
    prev = None
    for p in range(1, 101):
        s = o.clip_scale_fp16(amax, p).astype(np.float64)
        exact = (p / 100) * amax.astype(np.float64) / 7
        big = exact > 2 ** -14  # normal float16 range
        assert np.all(np.abs(s[big] - exact[big]) <= exact[big] * 2 ** -10.9)
        if prev is not None:
            assert np.all(s >= prev)
        prev = s
    assert np.array_equal(o.clip_scale_fp16(amax, 100).view(np.uint16), o.sym_scale_fp16(amax).view(np.uint16))


def pin_clip_exact_bruteforce(seed=22):
    """Exact rational brute force of the search on small matrices: codes by exact
    round-half-even of w/s16 clipped to +-7, errors as exact rationals, smallest
    error with ties to the larger percent."""
    o = _orc()
    for g, pmin, N, K in ((32, 85, 6, 96), (64, 90, 3, 128)):
        W = synth.weight(N, K, seed=seed + g)
        W[0, :g] = np.float16(0)                              # zero group: every error 0 -> p = 100
        W[1, :g] = np.float16(7 * 2.0 ** -4) * np.where(np.arange(g) % 2, 1, -1).astype(np.float16)  # exact at p = 100
        q, s, p = o.quantize_sym_clip(W, g, pmin)
        Wg = W.reshape(N, -1, g)
        for n in range(N):
            for j in range(Wg.shape[1]):
                w = [Fraction(float(v)) for v in Wg[n, j]]
                amax = np.abs(Wg[n, j]).max()
                best = None
                for pc in range(pmin, 101):
                    s16 = o.clip_scale_fp16(amax, pc)
                    sf = Fraction(float(s16))
                    codes = [0] * g if sf == 0 else [max(-7, min(7, _round_half_even(v / sf))) for v in w]
                    err = sum((sf * c - v) ** 2 for c, v in zip(codes, w))
                    if best is None or err <= best[0]:
                        best = (err, pc, codes, s16)
                assert int(p[n, j]) == best[1], (n, j, int(p[n, j]), best[1])
                assert q[n, j * g:(j + 1) * g].tolist() == best[2]
                assert s[n, j].view(np.uint16) == best[3].view(np.uint16)
        assert p[0, 0] == 100 and s[0, 0] == 0 and p[1, 0] == 100


def pin_clip_scale_steps_exact(n_amax=10_000, seed=63):
    """Reading C2's scale, each rounding step redone in exact integer arithmetic for
    every percent p in 1..100 and 10^4 float16 amax (all normal and subnormal
    binades): alpha = fl32(p / 100), a = fl32(fl32(amax) * alpha), a = max(a, fl32(1e-12)),
    s16 = fp16(fl32(a / 7)) ([ARG] section 三.2 with the RTN scale of [YBB] section 二)."""
    o = _orc()
    r = np.random.default_rng(seed)
    bits = np.concatenate([r.integers(1, 0x7BFF, size=n_amax - 6, endpoint=True),
                           [0x0001, 0x0400, 0x3C00, 0x4700, 0x7BFF, 0x0000]]).astype(np.uint16)
    amax = bits.view(np.float16)
    _, Ma, Ea = xr.decode_fp16(amax)
    # fl32(1e-12): 1e-12 = 2^-12 / 5^12, rounded once
    Qe, Te = xr.round_to(*xr.divide(np.array([1]), np.array([-12]), 5 ** 12), xr.FP32)
    eps = xr.to_float64(Qe, Te)[0]
    assert eps == float(np.float32(1e-12))  # the literal as a float32 constant takes the same value
    for p in range(1, 101):
        Qa, Ta = xr.round_to(*xr.divide(np.array([p]), np.array([0]), 100), xr.FP32)
        Mp, Ep = xr.multiply(Ma, Ea, Qa[0], Ta[0])
        Qm, Tm = xr.round_to(Mp, Ep, False, xr.FP32)
        small = xr.to_float64(Qm, Tm) < eps
        Qm = np.where(small, Qe[0], Qm)
        Tm = np.where(small, Te[0], Tm)
        Q32, T32 = xr.round_to(*xr.divide(Qm, Tm, 7), xr.FP32)
        Q16, T16 = xr.round_to(Q32, T32, False, xr.FP16)
        got = o.clip_scale_fp16(amax, p).astype(np.float64)
        exp = xr.to_float64(Q16, T16)
        assert np.array_equal(got, exp), (p, np.flatnonzero(got != exp)[:5])


def pin_clip_never_worse_than_rtn(seed=24):
    """Per group, the chosen codes reconstruct the weights at least as well as RTN's
    (alpha = 1 is one of the candidates), codes stay in -7..7, and Gaussian weights
    at g = 128 lose much of their error (about a fifth)."""
    o = _orc()
    W = synth.weight(64, 1024, seed=seed)
    for g in (32, 128):
        q, s, p = o.quantize_sym_clip(W, g, 80)
        assert q.min() >= -7 and q.max() <= 7 and p.min() >= 80 and p.max() <= 100
        q0, s0 = o.quantize_sym(W, g)
        e = (o.dequant_sym(q, s, g) - W.astype(np.float64)) ** 2
        e0 = (o.dequant_sym(q0, s0, g) - W.astype(np.float64)) ** 2
        eg = e.reshape(64, -1, g).sum(axis=2)
        e0g = e0.reshape(64, -1, g).sum(axis=2)
        assert np.all(eg <= e0g)
        if g == 128:
            assert eg.sum() < 0.9 * e0g.sum()


def pin_clip_gaussian_range():
    """[ARG] section 三.2: for Gaussian weights the MSE-optimal 4-bit range is about
    2.5-3 sigma while the maximum sits at 4-5 sigma. Large Gaussian groups searched
    from 0.4 amax choose a range of 2.3-3.1 sigma (2.48 measured)."""
    o = _orc()
    W = synth.weight(32, 8192, seed=3)
    g = 4096
    q, s, p = o.quantize_sym_clip(W, g, 40)
    Wg = W.astype(np.float64).reshape(32, -1, g)
    sig = Wg.std(axis=2)
    amax = np.abs(Wg).max(axis=2)
    chosen = p / 100 * amax / sig
    assert 3.5 < (amax / sig).mean() < 4.5
    assert 2.3 < chosen.mean() < 3.1


# ------------------------------------- per-channel INT8 RTN (W8A16, oracle/w8.py)


def pin_w8_outlier_example():
    """[ARG] section 七.1: a vector holding one 1000 among ones has the INT8 step
    1000/127 (about 8), and every other element quantizes to zero."""
    o = _orc()
    W = np.ones((1, 64), dtype=np.float16)
    W[0, 5] = np.float16(1000)
    q, s = o.quantize_w8(W)
    assert abs(float(s[0]) - 1000 / 127) <= (1000 / 127) * 2 ** -11 and 7.8 < float(s[0]) < 8.0
    assert q[0, 5] == 127 and np.count_nonzero(q) == 1
    assert o.dequant_w8(q, s)[0, 5] == 127 * float(s[0])


def pin_w8_clipping_example():
    """[IOC] section 1.2: W = 1000 against the INT8 range [-127, 127] at scale 1
    saturates at 127, a clipping error of 873."""
    o = _orc()
    W = np.array([[1000.0, -1000.0, 126.0]], dtype=np.float16)
    q = o.w8_codes(W, np.array([1.0], dtype=np.float16))
    assert q.tolist() == [[127, -127, 126]]
    assert float(W[0, 0]) - o.dequant_w8(q, np.array([1.0], dtype=np.float16))[0, 0] == 873.0


def pin_w8_hand_rows():
    """Rows whose amax is 127 * 2^k have an exact scale 2^k; codes worked by hand,
    ties to even: 254 -> 127, 1 -> 0.5 -> 0, -3 -> -1.5 -> -2, 128 -> 64, 5 -> 2.5 -> 2."""
    o = _orc()
    W = np.array([[254.0, 1.0, -3.0, 128.0, 5.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0],
                  [-0.4960938, 0.25, 0.0058594, -0.0058594, 0.0]], dtype=np.float16)
    q, s = o.quantize_w8(W)
    assert s.tolist() == [2.0, 0.0, float(np.float16(0.4960938) / np.float16(127))]
    assert q[0].tolist() == [127, 0, -2, 64, 2]
    assert q[1].tolist() == [0, 0, 0, 0, 0]           # W3: zero row -> codes 0, scale 0
    # row 2: amax = 127 * 2^-8 exactly, s = 2^-8: 0.25 -> 64, +-0.0058594 (1.5 * 2^-8) -> +-2
    assert float(s[2]) == 2.0 ** -8 and q[2].tolist() == [-127, 64, 2, -2, 0]


def pin_w8_scale_exhaustive():
    """fp16(fp32(a)/127) is the correctly rounded a/127 for every float16 a >= 0, and
    the quick code example's clamp of amax at 1e-6 changes no float16 scale (W1)."""
    o = _orc()
    a = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    s = o.w8_scale_fp16(a)
    assert np.array_equal(s.view(np.uint16), (a.astype(np.float64) / 127.0).astype(np.float16).view(np.uint16))
    assert np.array_equal(s.view(np.uint16), o.w8_scale_fp16(a, eps=1e-6).view(np.uint16))
    for ai, si in zip(a[1::89], s[1::89]):
        v = Fraction(float(ai)) / 127
        d = abs(v - Fraction(float(si)))
        for nb in (np.nextafter(si, np.float16(0)), np.nextafter(si, np.float16(np.inf))):
            dn = abs(v - Fraction(float(nb)))
            # a tie goes to the even significand
            assert d < dn or (d == dn and (si.view(np.uint16) & 1) == 0)


def pin_w8_code_decision_exact(n_scales=60, seed=31):
    """rint of the IEEE float32 quotient equals the exact rational decision for every
    float16 w with |w| <= amax of a row whose scale is s16 (W2)."""
    o = _orc()
    r = np.random.default_rng(seed)
    all16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    all16 = np.concatenate([all16, -all16[1:]])
    tried = 0
    for b in r.integers(0x0200, 0x5400, size=n_scales).astype(np.uint16):
        s16 = np.array([b], dtype=np.uint16).view(np.float16)[0]
        amax = np.float16(127 * float(s16))
        if not np.isfinite(amax) or o.w8_scale_fp16(np.array([amax]))[0] != s16:
            continue
        tried += 1
        w = all16[np.abs(all16.astype(np.float64)) <= float(amax)]
        sv = float(s16)
        q32 = np.clip(np.rint(w.astype(np.float32) / np.float32(sv)), -127, 127)
        q64 = np.clip(np.rint(w.astype(np.float64) / sv), -127, 127)
        assert np.array_equal(q32, q64), sv
        near = np.abs(np.abs(w.astype(np.float64) / sv) % 1.0 - 0.5) < 1e-9
        for wi, qi in zip(w[near], q64[near]):
            assert qi == max(-127, min(127, _round_half_even(Fraction(float(wi)) / Fraction(sv))))
        K = 256
        n_full = (w.size // (K - 1)) * (K - 1)
        rows = w[:n_full].reshape(-1, K - 1)
        Wm = np.concatenate([np.full((rows.shape[0], 1), amax, dtype=np.float16), rows], axis=1)
        q, s_or = o.quantize_w8(Wm)
        assert np.all(s_or == s16)
        assert np.array_equal(q[:, 1:].astype(np.float64).ravel(), q64[:n_full])
    assert tried >= 20


def pin_w8_invariants(seed=32):
    """[ARG] section 七.5: the INT8 step is absolute, every error within s/2; codes
    stay in -127..127 (never -128, also under subnormal scales), the row maximum maps
    to +-127, and the map is odd."""
    o = _orc()
    W = synth.weight(64, 2048, seed=seed)
    W[3] *= np.float16(1e-3)                     # amax ~1e-4: scale near the float16 subnormals
    W[4] = np.float16(0)
    W[4, 7] = np.float16(-1e-5)                  # scale a subnormal far below amax/127
    W[4, 9] = np.float16(9e-6)
    q, s = o.quantize_w8(W)
    assert q.min() >= -127 and q.max() <= 127
    assert q[4, 7] == -127 and q[4, 9] == 127
    err = np.abs(o.dequant_w8(q, s) - W.astype(np.float64))
    normal = s.astype(np.float64) >= 2.0 ** -14
    assert np.all(err[normal] <= s.astype(np.float64)[normal, None] / 2)
    am = np.abs(W).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), am])[normal] == 127)
    qn, sn = o.quantize_w8(-W)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def pin_w8_noise_model(N=512, K=4096, seed=33):
    """[ARG] section 三.1: uniform noise Delta^2/12 per weight; the row maximum is
    reproduced exactly, so the mean over rows of ((K-1)/K) s^2/12 (within 1%)."""
    o = _orc()
    W = synth.weight(N, K, seed=seed)
    q, s = o.quantize_w8(W)
    mse = o.quant_mse(W, o.dequant_w8(q, s))
    model = float(np.mean(s.astype(np.float64) ** 2)) / 12 * (K - 1) / K
    assert abs(mse / model - 1) < 0.01, mse / model
    # and INT8 per-channel beats INT4 at g = 128 by more than 50x (ARG section 四.3: nearly lossless)
    q4, s4 = o.quantize_sym(W, 128)
    assert o.quant_mse(W, o.dequant_sym(q4, s4, 128)) > 50 * mse


def pin_w8_layout_hand_positions():
    """Single codes planted at hand-computed device positions of the W8 layout."""
    o = _orc()
    N, K = 40, 352
    sh = o.w8_device_shapes(N, K)
    assert (sh["Np"], sh["Kp"], sh["S"], sh["code_bytes"]) == (48, 384, 3, 48 * 384)
    # (n, k, byte) from the spec, ((t*S + s)*2 + h)*1024 + (r + 16c)*16 + 8m + e:
    #   n=17,k=200: t=1 r=1 s=1 h=1 m=0 c=1 e=0 -> ((1*3+1)*2+1)*1024 + 17*16 + 0 + 0 = 9488
    #   n=0,k=1:    e=1 -> 1
    #   n=15,k=127: t=0 r=15 s=0 h=1 m=1 c=3 e=7 -> 1024 + 63*16 + 8 + 7 = 2047
    #   n=39,k=350: t=2 r=7 s=2 h=1 m=0 c=3 e=6 -> ((2*3+2)*2+1)*1024 + 55*16 + 0 + 6 = 18294
    for n, k, byte in ((17, 200, 9488), (0, 1, 1), (15, 127, 2047), (39, 350, 18294)):
        q = np.zeros((N, K), dtype=np.int64)
        q[n, k] = -5
        dev = o.w8_codes_to_device(q)
        assert dev[byte] == 123, (n, k)
        assert np.all(np.delete(dev, byte) == 128)
        assert np.array_equal(o.w8_codes_from_device(dev, N, K), q.astype(np.int8))
    r = np.random.default_rng(3)
    for N, K in ((16, 128), (33, 96), (5, 32), (48, 1024)):
        q = r.integers(-127, 128, size=(N, K))
        dev = o.w8_codes_to_device(q)
        assert np.array_equal(o.w8_codes_from_device(dev, N, K), q.astype(np.int8))
        assert np.array_equal(np.sort(dev[dev != 128]), np.sort((q + 128).ravel()[(q != 0).ravel()]))
    assert o.w8_scales_to_device(np.array([1, 2, 3], dtype=np.float16), 3).tolist() == [1, 2, 3] + [0] * 13


def pin_w8_product_bruteforce(seed=34):
    """Exact rational y = sum_k x * q * s over the codes (pure Python) against the oracle."""
    o = _orc()
    for B, N, K in ((1, 5, 32), (3, 17, 64), (2, 4, 200)):
        W = synth.weight(N, K, seed=seed + N)
        x = synth.activation(B, K, seed=seed + K)
        q, s = o.quantize_w8(W)
        rows = np.arange(N)[::-1]
        y = o.gemm_w8_rows(x, q, s, rows)
        for b in range(B):
            for i, n in enumerate(rows):
                ex = sum(Fraction(float(x[b, k])) * Fraction(float(s[n])) * int(q[n, k]) for k in range(K))
                assert abs(y[b, i] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


# ------------------------------- act-order groups with g_idx (oracle/actorder.py)


def pin_actorder_constant_h_is_rtn(seed=41):
    """Equal H_ii everywhere keeps the channel order: act-order is plain RTN, g_idx = k // g."""
    o = _orc()
    for g in (32, 128):
        W = synth.weight(24, 512, seed=seed + g)
        q, s, gi = o.quantize_sym_actorder(W, g, np.ones(512))
        q0, s0 = o.quantize_sym(W, g)
        assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))
        assert np.array_equal(gi, np.arange(512) // g)


def pin_actorder_hand_example():
    """K = 8, g = 4 worked by hand. h = [0.1, 5, 0.3, 2, 2, 0.2, 9, 2]: descending
    order 6, 1, 3, 4 | 7, 2, 5, 0 (the three-way tie at 2 keeps channels 3 and 4
    before 7, across the group boundary), so
    g_idx = [1, 0, 1, 0, 0, 1, 0, 1]. Row [0.5, -7, 1, 3.5, 2, -0.25, 0.75, 3.5]:
    group 0 {-7, 3.5, 2, 0.75} has amax 7, scale 1, codes -7, 4 (tie to even), 2, 1;
    group 1 {0.5, 1, -0.25, 3.5} has amax 3.5, scale 0.5, codes 1, 2, 0 (-0.5 to even), 7."""
    o = _orc()
    h = np.array([0.1, 5, 0.3, 2, 2, 0.2, 9, 2])
    assert o.actorder_order(h).tolist() == [6, 1, 3, 4, 7, 2, 5, 0]
    W = np.array([[0.5, -7, 1, 3.5, 2, -0.25, 0.75, 3.5]], dtype=np.float16)
    q, s, gi = o.quantize_sym_actorder(W, 4, h)
    assert gi.tolist() == [1, 0, 1, 0, 0, 1, 0, 1]
    assert s.tolist() == [[1.0, 0.5]]
    assert q.tolist() == [[1, -7, 2, 4, 2, 0, 1, 7]]
    assert o.dequant_gidx(q, s, gi).tolist() == [[0.5, -7, 1, 4, 2, 0, 1, 3.5]]
    q0, _ = o.quantize_sym(W, 4)                  # contiguous groups give other codes
    assert q0.tolist() != q.tolist()


def pin_actorder_gidx_structure(seed=42):
    """Every group holds exactly g channels, and every channel of group j has H_ii at
    least that of every channel of group j + 1."""
    o = _orc()
    r = np.random.default_rng(seed)
    for K, g in ((256, 32), (1024, 128), (384, 128)):
        h = r.lognormal(size=K)
        h[::7] = h[0]                               # ties
        gi = o.actorder_gidx(h, g)
        assert np.array_equal(np.bincount(gi, minlength=K // g), np.full(K // g, g))
        for j in range(K // g - 1):
            assert h[gi == j].min() >= h[gi == j + 1].max()


def pin_actorder_channel_relabelling(seed=43):
    """Relabelling the input channels of W and h together relabels the codes and leaves
    the scales unchanged (groups follow the H_ii values, not the positions)."""
    o = _orc()
    r = np.random.default_rng(seed)
    N, K, g = 16, 512, 64
    W = synth.weight(N, K, seed=seed)
    h = r.permutation(K).astype(np.float64)        # distinct values: no ties
    sigma = r.permutation(K)
    q, s, gi = o.quantize_sym_actorder(W, g, h)
    q2, s2, gi2 = o.quantize_sym_actorder(np.ascontiguousarray(W[:, sigma]), g, h[sigma])
    assert np.array_equal(q2, q[:, sigma]) and np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(gi2, gi[sigma])


def pin_actorder_outlier_columns():
    """With the 41 outlier input channels first in the order (largest H_ii) they share
    group 0, and every other group keeps a small scale: on the ordinary channels the
    weight error falls well below contiguous RTN's, where most groups hold an outlier;
    the outliers themselves now share one coarse scale and carry more error."""
    o = _orc()
    W, cols = synth.heavy_tailed_weight(64, 4096, seed=5)
    h = np.ones(4096)
    h[cols] = 50.0
    q, s, gi = o.quantize_sym_actorder(W, 128, h)
    assert np.all(gi[cols] == 0) and np.count_nonzero(gi == 0) == 128
    ordinary = np.ones(4096, dtype=bool)
    ordinary[cols] = False
    q0, s0 = o.quantize_sym(W, 128)
    e_ao = (o.dequant_gidx(q, s, gi) - W.astype(np.float64)) ** 2
    e_rtn = (o.dequant_sym(q0, s0, 128) - W.astype(np.float64)) ** 2
    assert e_ao[:, ordinary].mean() < 0.25 * e_rtn[:, ordinary].mean()
    assert e_ao[:, ~ordinary].mean() > e_rtn[:, ~ordinary].mean()


def pin_actorder_product_bruteforce(seed=44):
    """Exact rational y with each channel's scale looked up by hand from its group."""
    o = _orc()
    r = np.random.default_rng(seed)
    for B, N, K, g in ((2, 5, 64, 16), (1, 9, 96, 32)):
        W = synth.weight(N, K, seed=seed + N)
        x = synth.activation(B, K, seed=seed + K)
        h = r.lognormal(size=K)
        q, s, gi = o.quantize_sym_actorder(W, g, h)
        rank = sorted(range(K), key=lambda k: (-h[k], k))
        group_of = {k: i // g for i, k in enumerate(rank)}
        y = o.gemm_gidx_rows(x, q, s, gi, np.arange(N))
        for b in range(B):
            for n in range(N):
                ex = sum(Fraction(float(x[b, k])) * Fraction(float(s[n, group_of[k]])) * int(q[n, k]) for k in range(K))
                assert abs(y[b, n] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


# --------------------------------------------- INT4 KV cache (oracle/kv.py)


def pin_kv_bytes_per_token():
    """[YBB] section 七: Llama-3-70B's K and V take 2 * 80 * 8 * 128 * 2 = 327,680 bytes per
    token in BF16; INT4 with one float16 scale per 128 channels takes 2 * 80 * 8 * (64 + 2)."""
    o = _orc()
    assert o.kv_bytes_per_token(80, 8, 128) == 327_680
    assert o.kv_bytes_per_token(80, 8, 128, bits=4, group=128) == 84_480
    assert abs(327_680 / 84_480 - 3.879) < 1e-3


def pin_kv_hand_token():
    """One token, head_dim 16, group 8, worked by hand: group 0 has amax 7 (scale 1),
    codes 7, -4 (tie to even), 0, 2 (tie), 2 (tie), -7, 0, 1; group 1 has amax 0.875
    (scale 0.125), codes 1, -2, 7, 0, -7, 3, 4 (tie 3.5), 0; packed low nibble first."""
    o = _orc()
    K = np.zeros((1, 1, 1, 16), dtype=np.float16)
    K[0, 0, 0, :8] = [7, -3.5, 0.5, 1.5, 2.5, -7, 0, 1]
    K[0, 0, 0, 8:] = [0.125, -0.25, 0.875, 0.0, -0.875, 0.375, 0.4375, 0.0]
    q, s = o.quantize_kv_int4(K, 8)
    assert s.tolist() == [[[[1.0, 0.125]]]]
    assert q[0, 0, 0].tolist() == [7, -4, 0, 2, 2, -7, 0, 1, 1, -2, 7, 0, -7, 3, 4, 0]
    p = o.pack_kv_int4(q)
    assert p.shape == (1, 1, 1, 8)
    assert p[0, 0, 0].tolist() == [0xC7, 0x20, 0x92, 0x10, 0xE1, 0x07, 0x39, 0x04]
    assert o.dequant_kv_int4(q, s, 8)[0, 0, 0, 8:].tolist() == [0.125, -0.25, 0.875, 0, -0.875, 0.375, 0.5, 0]


def pin_kv_invariants(seed=51):
    """Per group: the amax element maps to +-7, every error is within s/2, codes stay in
    -7..7 (never -8) for random K; tokens are quantized independently (the scales follow
    the token, as a cache appended one token at a time needs)."""
    o = _orc()
    r = np.random.default_rng(seed)
    K = (r.standard_normal((2, 4, 33, 128)) * r.lognormal(size=(1, 4, 33, 1))).astype(np.float16)
    for g in (32, 64, 128):
        q, s = o.quantize_kv_int4(K, g)
        assert q.min() >= -7 and q.max() <= 7
        err = np.abs(o.dequant_kv_int4(q, s, g) - K.astype(np.float64))
        assert np.all(err <= np.repeat(s.astype(np.float64), g, axis=-1) / 2 + 1e-12)
        Kg = np.abs(K.reshape(2, 4, 33, 128 // g, g).astype(np.float64))
        qg = np.abs(q.reshape(2, 4, 33, 128 // g, g))
        hit = np.take_along_axis(qg, Kg.argmax(axis=-1)[..., None], axis=-1)
        assert np.all(hit == 7)
        q1, s1 = o.quantize_kv_int4(np.ascontiguousarray(K[:, :, 5:6]), g)
        assert np.array_equal(q1, q[:, :, 5:6]) and np.array_equal(s1.view(np.uint16), s[:, :, 5:6].view(np.uint16))


def pin_kv_attention_sink(seed=52):
    """[YBB] section 七: attention sinks give the first tokens' K abnormally large values.
    With scales per token and head, the other tokens' codes and scales do not change."""
    o = _orc()
    r = np.random.default_rng(seed)
    K = r.standard_normal((1, 8, 64, 128)).astype(np.float16)
    Ks = K.copy()
    Ks[:, :, :4] *= np.float16(100)
    q, s = o.quantize_kv_int4(K, 128)
    qs, ss = o.quantize_kv_int4(Ks, 128)
    assert np.array_equal(q[:, :, 4:], qs[:, :, 4:]) and np.array_equal(s[:, :, 4:], ss[:, :, 4:])
    assert np.all(ss[:, :, :4].astype(np.float64) > 50 * s[:, :, :4].astype(np.float64))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
