"""Per-output-channel symmetric INT8 RTN (W8A16), its device layout and product.

Test infrastructure only (see the package docstring for who may import it).

Formulas followed:
  * symmetric INT8, one scale per output channel (row of W [out, in]):
    s = row amax / 127, q = clamp(round(w / s), -127, 127), w_hat = q * s
    [CH, the closing quick code example (per_channel_int8_quant); IOC section 2.1,
     symmetric INT8 with range [-127, 127]; WIKI section 7.4.1.1, s = max|x| / 127;
     ARG section 四.3, INT8 per-channel RTN is the W8A16 default]
  * the product keeps 16-bit activations and multiplies them with the
    dequantized weights, y = x . w_hat^T [ARG section 二.3].

Readings (where the pages are silent, ambiguous or disagree):
  W1 Scale bits: s16 = float16_rne(float32(amax) / 127.0f), the rounding of a
     float16 tensor division (as R2 for INT4). The quick code example clamps
     amax at 1e-6 first; that changes no float16 scale (any amax below 1e-6
     gives a quotient below half the smallest float16 subnormal either way),
     which a test checks exhaustively.
  W2 Code decision: round half to even of the IEEE float32 quotient
     float32(w) / float32(s16), clamped to [-127, 127] (CH and IOC section 2.1;
     WIKI section 7.4.1.1 names [-128, 127] as the target range but its scale
     max/127 never reaches -128). A test shows the float32 decision equals the
     exact rational one for every code.
  W3 s16 == 0 (all-zero row, or one whose amax/127 underflows float16): every
     code 0 (the page's division would give 0/0).
  W4 Scales are float16, one per row, like the INT4 path's group scales.
  W5 Non-finite weights are rejected (ValueError).

Device layout (this project's own; the pages prescribe none), written from its
specification independently of the library's implementation:

  Np = ceil(N/16)*16 rows, Kp = ceil(K/128)*128 input channels, S = Kp/128.
  Code (n, k) with t = n // 16, r = n % 16, s = k // 128, h = (k % 128) // 64,
  m = (k % 64) // 32, c = (k % 32) // 8, e = k % 8 is the byte at
      ((t*S + s)*2 + h)*1024 + (r + 16*c)*16 + 8*m + e
  holding q + 128 (offset binary). Padding positions hold 128 (code 0).
  Scales: float16 [Np], padding rows 0.
"""

from __future__ import annotations

import numpy as np

from .rtn import _check_fp16_matrix

QMAX_W8 = 127
TILE_ROWS = 16
SUPER_K = 128


def w8_scale_fp16(amax16, eps: float | None = None) -> np.ndarray:
    """s16 = float16(float32(amax) / 127) (W1); eps, if given, clamps amax from below first."""
    a32 = np.asarray(amax16, dtype=np.float16).astype(np.float32)
    if eps is not None:
        a32 = np.maximum(a32, np.float32(eps))
    return (a32 / np.float32(QMAX_W8)).astype(np.float16)


def w8_codes(W16, s16) -> np.ndarray:
    """q = clamp(rint(fp32(w) / fp32(s16[row])), -127, 127), 0 where s16 == 0 (W2, W3)."""
    W = _check_fp16_matrix(W16)
    s32 = np.asarray(s16, dtype=np.float16).astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = W.astype(np.float32) / s32
    q = np.clip(np.rint(quot), -QMAX_W8, QMAX_W8)
    return np.where(s32 == 0, 0.0, q).astype(np.int8)


def quantize_w8(W16):
    """Per-row symmetric INT8 RTN of a float16 [N, K] matrix.

    Steps, in the order of the CH quick code example:
      1. amax = max |w| over each row (exact in float16);
      2. s16 = fp16(fp32(amax) / 127) (W1);
      3. q = clamp(rint(fp32(w) / fp32(s16)), -127, 127), 0 where s16 == 0 (W2, W3).
    Returns (q int8 [N, K], s16 float16 [N]).
    """
    W = _check_fp16_matrix(W16)
    amax = np.abs(W).max(axis=1)
    s16 = w8_scale_fp16(amax)
    return w8_codes(W, s16), s16


def dequant_w8(q, s16) -> np.ndarray:
    """w_hat = q * s, exact in float64 (the quick code example's w_hat)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s16, dtype=np.float64)[:, None]


def gemm_w8_rows(x16, q, s16, rows) -> np.ndarray:
    """y[:, rows] = x . w_hat[rows]^T in float64 (the plain definition, ARG section 二.3)."""
    rows = np.asarray(rows, dtype=np.int64)
    x = np.asarray(x16, dtype=np.float64)
    w = dequant_w8(np.asarray(q)[rows], np.asarray(s16)[rows])
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("shapes must be x [B, K] and q [N, K]")
    return x @ w.T


def w8_device_shapes(N: int, K: int) -> dict:
    Np = -(-N // TILE_ROWS) * TILE_ROWS
    Kp = -(-K // SUPER_K) * SUPER_K
    return {"Np": Np, "Kp": Kp, "S": Kp // SUPER_K, "code_bytes": Np * Kp}


def _w8_device_position(N: int, K: int):
    sh = w8_device_shapes(N, K)
    n = np.arange(sh["Np"], dtype=np.int64)[:, None]
    k = np.arange(sh["Kp"], dtype=np.int64)[None, :]
    t, r = n // TILE_ROWS, n % TILE_ROWS
    s, h = k // SUPER_K, (k % SUPER_K) // 64
    m, c, e = (k % 64) // 32, (k % 32) // 8, k % 8
    return ((t * sh["S"] + s) * 2 + h) * 1024 + (r + 16 * c) * 16 + 8 * m + e, sh


def w8_codes_to_device(q) -> np.ndarray:
    """Codes int [N, K] in -127..127 -> device bytes (offset binary, padding 128)."""
    q = np.asarray(q).astype(np.int64)
    if q.ndim != 2 or q.min(initial=0) < -QMAX_W8 or q.max(initial=0) > QMAX_W8:
        raise ValueError("codes must be 2-D in -127..127")
    N, K = q.shape
    pos, sh = _w8_device_position(N, K)
    full = np.full((sh["Np"], sh["Kp"]), 128, dtype=np.int64)
    full[:N, :K] = q + 128
    dev = np.empty(sh["code_bytes"], dtype=np.uint8)
    dev[pos.ravel()] = full.ravel()
    return dev


def w8_codes_from_device(dev, N: int, K: int) -> np.ndarray:
    """Device bytes -> codes int8 [N, K] (inverse of w8_codes_to_device on the valid region)."""
    dev = np.asarray(dev, dtype=np.uint8)
    pos, sh = _w8_device_position(N, K)
    if dev.size != sh["code_bytes"]:
        raise ValueError("device buffer size does not match [N, K]")
    return (dev[pos].astype(np.int64)[:N, :K] - 128).astype(np.int8)


def w8_scales_to_device(s16, N: int) -> np.ndarray:
    """Scales float16 [N] -> device [Np] (padding 0)."""
    s16 = np.asarray(s16, dtype=np.float16)
    if s16.shape != (N,):
        raise ValueError("scales must be [N]")
    out = np.zeros(-(-N // TILE_ROWS) * TILE_ROWS, dtype=np.float16)
    out[:N] = s16
    return out
