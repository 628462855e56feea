"""IEEE round-to-nearest-even of exact dyadic values, written with integers only.

Test infrastructure for the pins: it re-derives the rounding steps the oracle
takes with numpy float32 / float16 casts, so a pin built on it does not reuse
the routine it checks. A value is carried as an integer significand M >= 0, an
exponent E (value = M * 2**E) and a sticky flag meaning "the true value lies
strictly above M * 2**E, below (M + 1) * 2**E". Rounding to a binary format of
p significand bits whose smallest last-bit exponent is emin_lsb (subnormals
included) follows IEEE 754 roundTiesToEven: integer shifts, a comparison of the
discarded bits with one half, ties to an even significand. numpy is used for
array integer arithmetic, for np.frexp on integers below 2**53 (exact: it only
reads the bit length) and for np.ldexp to hand results back as float64 (exact
for significands below 2**53).
"""

from __future__ import annotations

import numpy as np

# (significand bits p, smallest last-bit exponent, largest exponent of a finite value)
FP32 = (24, -149, 127)
FP16 = (11, -24, 15)


def bit_length(M):
    M = np.asarray(M, dtype=np.int64)
    _, e = np.frexp(M.astype(np.float64))  # M < 2**53: the conversion is exact
    return np.where(M == 0, 0, e).astype(np.int64)


def decode_fp16(a16):
    """float16 array -> (sign in {+1, -1}, M, E) with |a| = M * 2**E, from the bit fields."""
    b = np.asarray(a16, dtype=np.float16).view(np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1, 1)
    ex = (b >> 10) & 0x1F
    fr = b & 0x3FF
    if np.any(ex == 0x1F):
        raise ValueError("non-finite float16")
    M = np.where(ex == 0, fr, fr | 0x400)
    E = np.where(ex == 0, -24, ex - 25)
    return sign, M, E


def on_grid(a16, lsb=-24):
    """float16 array -> the signed integer a * 2**(-lsb) (every float16 is a multiple of 2**-24)."""
    sign, M, E = decode_fp16(a16)
    return sign * (M << (E - lsb))


def round_to(M, E, sticky, fmt):
    """Round M * 2**E (+ sticky) to the format; returns (Q, T) with the result Q * 2**T,
    or Q = -1 where it overflows to infinity."""
    p, emin_lsb, emax = fmt
    M = np.asarray(M, dtype=np.int64)
    E = np.broadcast_to(np.asarray(E, dtype=np.int64), M.shape)
    sticky = np.broadcast_to(np.asarray(sticky, dtype=bool), M.shape)
    nb = bit_length(M)
    T = np.maximum(E + nb - p, emin_lsb)
    shift = T - E
    if np.any((shift <= 0) & sticky & (M > 0)):
        raise ValueError("too few significand bits carried for a sticky value")
    exact = shift <= 0
    s = np.where(exact, 0, shift)
    Q = M >> s
    rem = M - (Q << s)
    half = np.where(exact, 0, np.int64(1) << np.maximum(s - 1, 0))
    up = ~exact & ((rem > half) | ((rem == half) & (sticky | ((Q & 1) == 1))))
    Q = np.where(exact, M << np.maximum(-shift, 0), Q + up)
    T = np.where(exact, E + np.minimum(shift, 0), T)
    Q = np.where(M == 0, 0, Q)
    # a carry out of the top bit leaves Q = 2**p, which is still exact; beyond the
    # largest finite value the result is infinite
    big = (Q > 0) & (bit_length(Q) + T > emax + 1)
    return np.where(big, -1, Q), T


def divide(M, E, d: int, extra: int = 61):
    """M * 2**E / d for a positive integer d, as (M', E', sticky) with at least
    `extra` - bit_length(M) more bits than M (enough for any format here)."""
    M = np.asarray(M, dtype=np.int64)
    k = np.maximum(extra - bit_length(M), 0)
    num = M << k
    return num // d, np.asarray(E, dtype=np.int64) - k, (num % d) != 0


def multiply(M1, E1, M2, E2):
    M = np.asarray(M1, dtype=np.int64) * np.asarray(M2, dtype=np.int64)
    if np.any(bit_length(np.where(M < 0, 0, M)) > 62):
        raise OverflowError("product too wide")
    return M, np.asarray(E1, dtype=np.int64) + np.asarray(E2, dtype=np.int64)


def to_float64(Q, T):
    """(Q, T) -> float64 (exact), +inf where Q == -1."""
    Q = np.asarray(Q, dtype=np.int64)
    v = np.ldexp(np.where(Q < 0, 0, Q).astype(np.float64), np.asarray(T, dtype=np.int64))
    return np.where(Q < 0, np.inf, v)


def rint_div(num, den):
    """Round-half-even of num / den for integer arrays, den > 0."""
    num = np.asarray(num, dtype=np.int64)
    den = np.asarray(den, dtype=np.int64)
    q = np.floor_divide(num, den)
    r = num - q * den
    twice = 2 * r
    return q + ((twice > den) | ((twice == den) & ((q & 1) == 1)))
