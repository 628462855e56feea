"""Clipping search for the symmetric INT4 group scale, written out from the pages.

Test infrastructure only (see the package docstring for who may import it).

[ARG] section 三.2 ("clipping vs rounding"): the range alpha that sets the step
Delta = alpha / 7 trades rounding error (a larger alpha widens every step) against
clipping error (a smaller alpha saturates the weights beyond it); every practical
quantizer searches a set of ranges, for example 0.8 to 1.0 times the maximum, and
keeps the one with the smallest error. The grid of section 三.1 is symmetric,
-(2^(b-1) - 1) .. 2^(b-1) - 1 = -7 .. 7 for INT4, so codes are clipped to +-7.

Steps, per group of g consecutive input channels of a row:
  1. amax = max |w| (exact in float16);
  2. for p = p_min .. 100: alpha_p = float32(p) / float32(100) (IEEE float32),
     s16_p = float16(float32(max(float32(amax) * alpha_p, 1e-12)) / 7) -- the RTN
     scale of rtn.py with the clipped range;
  3. q_p = clamp(rint(float32(w) / float32(s16_p)), -7, 7), q_p = 0 where s16_p == 0;
  4. err_p = sum over the group of (s16_p * q_p - w)^2;
  5. keep the p with the smallest err_p; equal errors go to the larger p (the
     smaller clip), so p_min = 100 -- and any group where clipping does not pay --
     is exactly RTN.

Readings (where the pages are silent, ambiguous or disagree):
  C1 The error is the weight reconstruction error of the group itself (the pages
     search "on calibration data"; weight-only RTN has none, and the squared
     weight error is the quantity section 三.2's formula writes out).
  C2 The candidates are alpha = p/100 for integer percent p from p_min to 100
     (the page's example range 0.8 .. 1.0 is p_min = 80); alpha_p, the clipped
     range and the scale are rounded as written in step 2.
  C3 Codes are clipped to -7 .. 7 (the symmetric grid of section 三.1). At p = 100
     this equals RTN's [-8, 7] clamp, which never produces -8 (|w / s16| < 7.5).
  C4 err_p is accumulated in float64: every difference s16_p * q_p - w is exact in
     float32 (both terms lie on float16 grids within a factor 2^4 of each other
     unless q_p = 0) and its square exact in float64; the sum is exact in any order
     when the group's nonzero magnitudes span less than 2^12, and otherwise rounds
     by at most ~2^-53 relative, which can only matter for two candidates whose
     errors agree to that precision (the kernel sums in another order).
"""

from __future__ import annotations

import numpy as np

from .rtn import _check_fp16_matrix, _group_view

CLIP_QMAX = 7


def clip_scale_fp16(amax16, percent: int) -> np.ndarray:
    """s16_p = float16(float32(max(float32(amax) * float32(p)/float32(100), 1e-12)) / 7) (step 2, C2)."""
    alpha = np.float32(percent) / np.float32(100)
    a32 = np.asarray(amax16, dtype=np.float16).astype(np.float32) * alpha
    a32 = np.maximum(a32, np.float32(1e-12))
    return (a32 / np.float32(CLIP_QMAX)).astype(np.float16)


def clip_codes(Wg16: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """q = clamp(rint(fp32(w) / fp32(s16)), -7, 7), 0 where s16 == 0 (step 3, C3).

    Wg16: float16 [..., g]; s16: float16 [...]."""
    s32 = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = Wg16.astype(np.float32) / s32
    q = np.clip(np.rint(quot), -CLIP_QMAX, CLIP_QMAX)
    return np.where(s32 == 0, 0.0, q)


def clip_errors(W16, g: int, min_percent: int = 80) -> np.ndarray:
    """err[p - min_percent, n, j] = sum_k (s16_p q_p - w)^2 over group j of row n (steps 2-4, C4)."""
    W = _check_fp16_matrix(W16)
    Wg = _group_view(W, g)
    amax = np.abs(Wg).max(axis=2)
    w64 = Wg.astype(np.float64)
    errs = []
    for p in range(min_percent, 101):
        s16 = clip_scale_fp16(amax, p)
        q = clip_codes(Wg, s16)
        d = s16.astype(np.float64)[..., None] * q - w64
        errs.append((d * d).sum(axis=2))
    return np.stack(errs)


def quantize_sym_clip(W16, g: int, min_percent: int = 80):
    """Group-wise symmetric INT4 with the clipping search of [ARG] section 三.2.

    Returns (q int8 [N, K] in -7..7, s16 float16 [N, K/g], percent int [N, K/g])."""
    if not 1 <= min_percent <= 100:
        raise ValueError("min_percent must be in 1..100")
    W = _check_fp16_matrix(W16)
    Wg = _group_view(W, g)
    errs = clip_errors(W, g, min_percent)
    # step 5: smallest error, ties to the larger percent -> argmin over the reversed axis
    rev = errs[::-1]
    best = rev.shape[0] - 1 - np.argmin(rev, axis=0)
    percent = best + min_percent
    amax = np.abs(Wg).max(axis=2)
    s16 = np.zeros(amax.shape, dtype=np.float16)
    for p in np.unique(percent):
        sel = percent == p
        s16[sel] = clip_scale_fp16(amax[sel], int(p))
    q = clip_codes(Wg, s16)
    return q.astype(np.int8).reshape(W.shape), s16, percent.astype(np.int64)
