"""Byte layouts of the quantized weights: the canonical packing and the device layout.

Test infrastructure only (see the package docstring).

Canonical packing ([WIKI] section 7.4.1.2 packs two INT4 codes into one byte
but does not define the order; ARG section 二.2 counts 4 bits per code):
    byte[n, i] = (c[n, 2i] & 0xF) | ((c[n, 2i+1] & 0xF) << 4)
i.e. the low nibble holds the even input channel. Symmetric codes are stored
as 4-bit two's complement, asymmetric codes (0..15) as they are.

Device layout (this project's own; the pages prescribe none). Written here
from its specification, independently of the library's implementation:

  Np = ceil(N/16)*16 rows, Kp = ceil(K/128)*128 input channels,
  S = Kp/128 super-blocks per row-tile.
  Code (n, k) with t = n // 16, r = n % 16, s = k // 128, m = (k % 128) // 32,
  c = (k % 32) // 8, e = k % 8 lives in
      byte  ((t*S + s)*64 + (r + 16*c))*16 + 4*m + p(e)//2,
      nibble p(e) % 2 of that byte (0 = low),
  where p(e) = e/2 for even e and 4 + (e-1)/2 for odd e.
  Nibble value: q + 8 for symmetric codes (offset binary), q for asymmetric.
  Padding positions (n >= N or k >= K) hold the value of code 0: 8 (symmetric)
  or 0 (asymmetric).

Per-group arrays (scales float16, asymmetric zeros uint8) in device layout are
[Np/16, Gp, 16] with Gp = Kp/g: element [t, j, r] = value for row 16t + r and
group j; padding (row >= N or j >= K/g) is 0.
"""

from __future__ import annotations

import numpy as np

TILE_ROWS = 16
SUPER_K = 128


def pack_canonical(c) -> np.ndarray:
    """Two codes per byte, low nibble = even input channel."""
    c = np.asarray(c).astype(np.int64)
    if c.ndim != 2 or c.shape[1] % 2:
        raise ValueError("codes must be 2-D with an even number of columns")
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_canonical(b, signed: bool = True) -> np.ndarray:
    """Inverse of pack_canonical; signed=True reads 4-bit two's complement."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8 if signed else np.uint8)


def device_shapes(N: int, K: int, g: int) -> dict:
    """Sizes of the device arrays for an [N, K] matrix with group size g."""
    Np = -(-N // TILE_ROWS) * TILE_ROWS
    Kp = -(-K // SUPER_K) * SUPER_K
    Gp = -(-Kp // g)
    return {
        "Np": Np,
        "Kp": Kp,
        "S": Kp // SUPER_K,
        "Gp": Gp,
        "code_bytes": Np * Kp // 2,
        "group_elems": Np * Gp,
    }


def _nibble_index(e: np.ndarray) -> np.ndarray:
    return np.where(e % 2 == 0, e // 2, 4 + (e - 1) // 2)


def _device_position(N: int, K: int):
    """Byte offset and nibble shift of every code position of the padded grid."""
    Kp = -(-K // SUPER_K) * SUPER_K
    Np = -(-N // TILE_ROWS) * TILE_ROWS
    S = Kp // SUPER_K
    n = np.arange(Np, dtype=np.int64)[:, None]
    k = np.arange(Kp, dtype=np.int64)[None, :]
    t, r = n // TILE_ROWS, n % TILE_ROWS
    s, m = k // SUPER_K, (k % SUPER_K) // 32
    c, e = (k % 32) // 8, k % 8
    p = _nibble_index(e)
    byte = ((t * S + s) * 64 + (r + 16 * c)) * 16 + 4 * m + p // 2
    shift = 4 * (p % 2)
    return byte, np.broadcast_to(shift, byte.shape), Np, Kp


def codes_to_device(q, symmetric: bool = True) -> np.ndarray:
    """Codes [N, K] (signed for symmetric, 0..15 for asymmetric) -> device bytes."""
    q = np.asarray(q).astype(np.int64)
    N, K = q.shape
    byte, shift, Np, Kp = _device_position(N, K)
    pad = 8 if symmetric else 0
    nib = np.full((Np, Kp), pad, dtype=np.int64)
    nib[:N, :K] = q + 8 if symmetric else q
    if nib.min() < 0 or nib.max() > 15:
        raise ValueError("codes out of the 4-bit range")
    dev = np.zeros(Np * Kp // 2, dtype=np.int64)
    lo = shift == 0
    dev[byte[lo]] = nib[lo]
    dev[byte[~lo]] |= nib[~lo] << 4
    return dev.astype(np.uint8)


def codes_from_device(dev, N: int, K: int, symmetric: bool = True) -> np.ndarray:
    """Device bytes -> codes [N, K] (inverse of codes_to_device on the valid region)."""
    dev = np.asarray(dev, dtype=np.uint8).astype(np.int64)
    byte, shift, Np, Kp = _device_position(N, K)
    if dev.size != Np * Kp // 2:
        raise ValueError("device buffer size does not match [N, K]")
    nib = (dev[byte] >> shift) & 0xF
    nib = nib[:N, :K]
    return (nib - 8).astype(np.int8) if symmetric else nib.astype(np.uint8)


def groupwise_to_device(a, N: int, K: int, g: int) -> np.ndarray:
    """Per-group array [N, K/g] -> device layout [Np/16, Gp, 16] (padding 0)."""
    a = np.asarray(a)
    sh = device_shapes(N, K, g)
    if a.shape != (N, K // g):
        raise ValueError("per-group array must be [N, K/g]")
    full = np.zeros((sh["Np"], sh["Gp"]), dtype=a.dtype)
    full[:N, : K // g] = a
    return np.ascontiguousarray(full.reshape(sh["Np"] // TILE_ROWS, TILE_ROWS, sh["Gp"]).transpose(0, 2, 1))


def groupwise_from_device(d, N: int, K: int, g: int) -> np.ndarray:
    """Inverse of groupwise_to_device on the valid region."""
    sh = device_shapes(N, K, g)
    d = np.asarray(d).reshape(sh["Np"] // TILE_ROWS, sh["Gp"], TILE_ROWS)
    full = d.transpose(0, 2, 1).reshape(sh["Np"], sh["Gp"])
    return np.ascontiguousarray(full[:N, : K // g])
