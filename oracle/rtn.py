"""Round-to-nearest (RTN) quantization, written out from the pages' formulas.

Test infrastructure only (see the package docstring for who may import it).

Formulas followed:
  * affine map  q = clamp(round(w/s) + z, qmin, qmax),  w_hat = s * (q - z)
    [CH section 1; YBB section 二, the displayed affine map; ARG section 二.2]
  * symmetric INT4, one scale per group of g consecutive input channels of a
    row: s = group amax / 7, q = clamp(round(w/s), -8, 7)
    [YBB section 二, quantize_per_group; ARG section 三.1, step alpha/7;
     WIKI section 7.4.1.2; CH section 1, range {-8..7}]
  * asymmetric uint4: s = (max - min)/15, z = round(-min/s),
    q = clamp(round(w/s) + z, 0, 15), w_hat = s*(q - z)
    [ARG section 二.2, integer-side zero point; WIKI section 7.4.1.1 with
     2^b - 1 = 15 for b = 4]

Readings (where the pages are silent or disagree):
  R1 The quotient divides by the *stored* float16 scale: the page's code
     quantizes and dequantizes with the same ``scale`` tensor, which is float16
     because W is.
  R2 Scale bits: s16 = float16_rne(float32(amax) / 7.0f). This is what an
     fp16 tensor division produces (computed in float32, rounded once to
     float16); an exhaustive test shows it equals the correctly rounded amax/7
     for every positive finite float16.
  R3 Code decision: round-half-to-even of the IEEE float32 quotient
     float32(w) / float32(s16). The page's own snippet rounds that quotient to
     float16 first; we do not (the kernel's precision decides, and a test shows
     the float32 decision equals the exact rational one).
  R4 All-zero (or scale-underflowing) group: s16 == 0 -> every code 0, scale 0.
     The page's clamp(min=1e-12) is a no-op in float16, so its code would divide
     by zero; code 0 is what its integer cast then yields.
  R5 Asymmetric scale bits: s16 = float16_rne(float32(float32(max) -
     float32(min)) / 15.0f); zero z = clamp(rint(-min / s16), 0, 15) (a 4-bit
     zero, as in the bits-per-weight count of ARG section 二.2); s16 == 0 ->
     q = z = 0.
  R6 Non-finite weights are rejected (ValueError).
"""

from __future__ import annotations

import numpy as np

QMIN_SYM, QMAX_SYM = -8, 7
QMAX_ASYM = 15


def rtn_scalar(w: float, s: float, qmin: int | None = None, qmax: int | None = None, z: int = 0):
    """One value through the affine map, exact (float64) arithmetic.

    Returns (q, w_hat, |w - w_hat|). With qmin = qmax = None no clamp is applied,
    which is how the worked example of [IOC] section 1.2 (3.14159 at scale 0.01)
    is stated: its code 314 lies outside the INT8 range printed beside it.
    """
    q = float(np.rint(np.float64(w) / np.float64(s))) + z
    if qmin is not None:
        q = max(q, qmin)
    if qmax is not None:
        q = min(q, qmax)
    w_hat = float(np.float64(s) * (q - z))
    return int(q), w_hat, abs(float(w) - w_hat)


def _check_fp16_matrix(W) -> np.ndarray:
    W = np.asarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise TypeError("W must be a 2-D float16 array [out_features, in_features]")
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds non-finite values")  # reading R6
    return W


def _group_view(W: np.ndarray, g: int) -> np.ndarray:
    n, k = W.shape
    if g <= 0 or k % g != 0:
        # [YBB] section 二 asserts in_features % group_size == 0.
        raise ValueError(f"in_features {k} is not a multiple of group size {g}")
    return W.reshape(n, k // g, g)


def sym_scale_fp16(amax16: np.ndarray, qmax: int = QMAX_SYM) -> np.ndarray:
    """s16 = float16(float32(max(amax, 1e-12)) / float32(qmax)) (readings R2, R4)."""
    a32 = np.maximum(np.asarray(amax16, dtype=np.float16).astype(np.float32), np.float32(1e-12))
    return (a32 / np.float32(qmax)).astype(np.float16)


def asym_scale_fp16(mn16: np.ndarray, mx16: np.ndarray, levels: int = QMAX_ASYM) -> np.ndarray:
    """s16 = float16(float32(float32(max) - float32(min)) / float32(15)) (reading R5)."""
    rng32 = np.asarray(mx16, dtype=np.float16).astype(np.float32) - np.asarray(mn16, dtype=np.float16).astype(np.float32)
    return (rng32 / np.float32(levels)).astype(np.float16)


def quantize_sym(W16, g: int):
    """Group-wise symmetric INT4 RTN of a float16 [N, K] matrix.

    Steps, in the order of [YBB] section 二:
      1. group amax = max |w| over each run of g input channels of a row;
      2. s16 = fp16(fp32(amax) / 7) (R2);
      3. q = clamp(rint(fp32(w) / fp32(s16)), -8, 7) (R1, R3), q = 0 where s16 == 0 (R4).
    Returns (q int8 [N, K], s16 float16 [N, K/g]).
    """
    W = _check_fp16_matrix(W16)
    Wg = _group_view(W, g)
    amax = np.abs(Wg).max(axis=2)                       # exact in float16
    s16 = sym_scale_fp16(amax)
    s32 = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = Wg.astype(np.float32) / s32               # IEEE float32 quotient
    q = np.clip(np.rint(quot), QMIN_SYM, QMAX_SYM)
    q = np.where(s32 == 0, 0.0, q)
    return q.astype(np.int8).reshape(W.shape), s16


def quantize_sym_exact(W, g: int, qmax: int = QMAX_SYM):
    """The same steps in exact float64 with an unrounded scale amax/qmax.

    Used for the pages' real-valued worked examples (the four-weight table of
    [ARG] section 六.2), which do not round the scale to float16.
    Returns (q int [N, K], s float64 [N, K/g]).
    """
    W = np.asarray(W, dtype=np.float64)
    Wg = _group_view(W, g)
    s = np.abs(Wg).max(axis=2) / qmax
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(Wg / s[..., None]), -qmax - 1, qmax)
    q = np.where(s[..., None] == 0, 0.0, q)
    return q.astype(np.int64).reshape(W.shape), s


def quantize_asym(W16, g: int):
    """Group-wise asymmetric uint4 RTN (reading R5).

    s16 = fp16(fp32(fp32(max) - fp32(min)) / 15); z = clamp(rint(-min/s16), 0, 15);
    q = clamp(rint(w/s16) + z, 0, 15); all quotients in IEEE float32.
    Returns (q uint8 [N, K] in 0..15, s16 float16 [N, K/g], z uint8 [N, K/g]).
    """
    W = _check_fp16_matrix(W16)
    Wg = _group_view(W, g)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    s16 = asym_scale_fp16(mn, mx)
    s32 = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.clip(np.rint(-mn.astype(np.float32) / s32), 0, QMAX_ASYM)
        z = np.where(s32 == 0, 0.0, z)
        quot = Wg.astype(np.float32) / s32[..., None]
    q = np.clip(np.rint(quot) + z[..., None], 0, QMAX_ASYM)
    q = np.where(s32[..., None] == 0, 0.0, q)
    return q.astype(np.uint8).reshape(W.shape), s16, z.astype(np.uint8)


def dequant_sym(q, s, g: int) -> np.ndarray:
    """w_hat = s * q, exact in float64 ([YBB] section 二, the dequantization check)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return q * np.repeat(s, g, axis=1)


def dequant_asym(q, s, z, g: int) -> np.ndarray:
    """w_hat = s * (q - z), exact in float64 ([ARG] section 二.2: subtract z, then scale)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    return (q - np.repeat(z, g, axis=1)) * np.repeat(s, g, axis=1)


def quant_mse(W, w_hat) -> float:
    """mean((w_hat - w)^2) over every element ([YBB] section 二)."""
    d = np.asarray(w_hat, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    return float(np.mean(d * d))
