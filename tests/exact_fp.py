"""Exact IEEE binary32 arithmetic on rationals, for pinning the oracle.

Every operation takes binary32 operands (as bit patterns), computes the exact
real result with ``fractions.Fraction`` (square roots with integer square
roots and a sticky bit) and rounds it once to binary32, round to nearest with
ties to even, with gradual underflow. This is what IEEE 754 defines each
operation to return, written out from that definition, so it shares nothing
with the C oracle except the definition itself.

Small formats (FP8 E4M3/E5M2, FP16) are encoded by brute force: the nearest of
all finite values of the format, taken from torch's CPU float8/float16 decode
tables (library routines), ties to the even code, saturating for FP8.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np
import torch

# ------------------------------------------------------------- binary32 ---


def bits_to_fraction(b: int) -> Fraction:
    """Exact value of a finite binary32 bit pattern."""
    sign = -1 if (b >> 31) & 1 else 1
    e = (b >> 23) & 0xFF
    m = b & 0x7FFFFF
    assert e != 0xFF, "non-finite operand"
    if e == 0:
        return sign * Fraction(m, 1 << 149)
    return sign * Fraction((1 << 23) | m) * Fraction(2) ** (e - 150)


def float_to_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_bits(x: Fraction, neg_zero: bool = False) -> int:
    """Round an exact rational to binary32 (RNE, subnormals, overflow to Inf)."""
    if x == 0:
        return 0x80000000 if neg_zero else 0
    sign = 1 if x < 0 else 0
    a = -x if sign else x
    e = max(_floor_log2(a), -126)
    q = Fraction(2) ** (e - 23)
    r = a / q
    n = r.numerator // r.denominator
    frac = r - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 1 << 24:
        e += 1
        n = 1 << 23
    if e > 127:
        return (sign << 31) | 0x7F800000
    if n < (1 << 23):
        return (sign << 31) | n
    return (sign << 31) | ((e + 127) << 23) | (n - (1 << 23))


def _rne_sqrt(x: Fraction) -> int:
    assert x >= 0
    if x == 0:
        return 0
    K = 400
    scaled = x * (Fraction(2) ** (2 * K))
    fl = scaled.numerator // scaled.denominator
    s = math.isqrt(fl)
    if Fraction(s * s) == scaled:
        return round_to_bits(Fraction(s, 1 << K))
    # sqrt lies strictly inside (s, s+1)/2^K; the midpoint of that interval
    # rounds the same way (no binary32 rounding boundary can fall inside an
    # interval this narrow around a square root of a binary32 value).
    return round_to_bits(Fraction(2 * s + 1, 1 << (K + 1)))


class F:
    """A binary32 value with exact IEEE operations (each result rounded once)."""

    __slots__ = ("b",)

    def __init__(self, b: int):
        self.b = b & 0xFFFFFFFF

    @staticmethod
    def of(x: float) -> "F":
        return F(float_to_bits(np.float32(x).item()))

    @property
    def q(self) -> Fraction:
        return bits_to_fraction(self.b)

    def __mul__(self, o: "F") -> "F":
        neg = ((self.b ^ o.b) >> 31) & 1
        return F(round_to_bits(self.q * o.q, neg_zero=bool(neg)))

    def __truediv__(self, o: "F") -> "F":
        neg = ((self.b ^ o.b) >> 31) & 1
        return F(round_to_bits(self.q / o.q, neg_zero=bool(neg)))

    def __neg__(self) -> "F":
        return F(self.b ^ 0x80000000)

    def sqrt(self) -> "F":
        return F(_rne_sqrt(self.q))

    @staticmethod
    def fma(a: "F", b: "F", c: "F") -> "F":
        exact = a.q * b.q + c.q
        if exact == 0:
            prod_neg = ((a.b ^ b.b) >> 31) & 1
            c_neg = (c.b >> 31) & 1
            return F(0x80000000 if (prod_neg and c_neg) else 0)
        return F(round_to_bits(exact))

    def __repr__(self):
        return "F(0x%08x)" % self.b


# --------------------------------------------------------- small formats ---

_TORCH_FP8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def fp8_table(fmt: int) -> np.ndarray:
    """float64 value of every code 0..255, from torch's CPU decode."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(_TORCH_FP8[fmt]).to(torch.float64).numpy()


def fp8_max(fmt: int) -> float:
    t = fp8_table(fmt)
    return float(np.nanmax(t[np.isfinite(t)]))


def brute_encode_fp8(x: Fraction, fmt: int, negative: bool) -> int:
    """Nearest finite code of the same sign (ties to the even code),
    saturating at +-max. ``negative`` carries the sign (also of zero)."""
    table = fp8_table(fmt)
    best = None
    for c in range(256):
        if ((c >> 7) & 1) != int(negative):
            continue
        v = table[c]
        if not np.isfinite(v):
            continue
        d = abs(Fraction(v) - x)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return best[1]


def brute_encode_f16(x: Fraction, negative: bool) -> int:
    """binary16 RNE of an exact value by search over the finite values near it."""
    v = float(x)  # only used to find the neighbourhood
    h = np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0]
    cands = set()
    base = int(h) & 0x7FFF
    for d in range(-2, 3):
        c = base + d
        if 0 <= c <= 0x7BFF:
            cands.add(c)
    best = None
    for c in sorted(cands):
        val = Fraction(np.array([c], np.uint16).view(np.float16).astype(np.float64)[0])
        d = abs(val - abs(x))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return (0x8000 if negative else 0) | best[1]


def f16_value(h: int) -> F:
    v = np.array([h], np.uint16).view(np.float16).astype(np.float32)[0]
    return F(float_to_bits(float(v)))


def fp8_value(code: int, fmt: int) -> F:
    return F(float_to_bits(float(np.float32(fp8_table(fmt)[code]))))
