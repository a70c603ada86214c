"""Brute-force MX reference used only to pin the oracle in tests.

It shares nothing with the oracle's arithmetic: it enumerates every code of an
element format (through the oracle's decode table, which is pinned on its own
against named values and torch's float8 casts), and rounds a value by looking
for its two neighbours in that list, in exact rational arithmetic.
"""
from __future__ import annotations

import bisect
import math
import struct
from fractions import Fraction

import numpy as np

FMT_NAMES = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8"]
FMT_BITS = [8, 8, 6, 6, 4, 8]


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def is_sub32(v: float) -> bool:
    b = f32_bits(v)
    return ((b >> 23) & 0xFF) == 0 and (b & 0x7FFFFF) != 0


class Grid:
    """All non-negative finite values of one element format with their codes."""

    def __init__(self, oracle, fmt: int):
        self.fmt = fmt
        self.is_int = fmt == 5
        vals = {}
        if self.is_int:
            for n in range(0, 128):
                vals[Fraction(n, 64)] = n
        else:
            nbits = FMT_BITS[fmt]
            for code in range(1 << (nbits - 1)):  # sign bit clear
                v = oracle.elem_value(fmt, code)
                if math.isfinite(v):
                    fv = Fraction(v)
                    assert fv not in vals
                    vals[fv] = code
        self.values = sorted(vals)
        self.codes = [vals[v] for v in self.values]
        self.maxnorm = self.values[-1]
        self.sign_bit = 0 if self.is_int else 1 << (FMT_BITS[fmt] - 1)
        # largest normal exponent: the binade holding the largest value
        self.emax = math.floor(math.log2(self.maxnorm)) if not self.is_int else 0

    def _neighbours(self, a: Fraction):
        i = bisect.bisect_left(self.values, a)
        if i < len(self.values) and self.values[i] == a:
            return i, i
        return i - 1, i

    def _signed(self, idx: int, neg: bool) -> int:
        code = self.codes[idx]
        if self.is_int:
            return (-code) & 0xFF if neg else code
        return code | (self.sign_bit if neg else 0)

    def nearest_even(self, y: Fraction, neg: bool) -> int:
        a = abs(y)
        if a >= self.maxnorm:
            return self._signed(len(self.values) - 1, neg)
        lo, hi = self._neighbours(a)
        if lo == hi:
            return self._signed(lo, neg)
        dl, dh = a - self.values[lo], self.values[hi] - a
        if dl < dh:
            pick = lo
        elif dh < dl:
            pick = hi
        else:  # tie: the code whose lowest bit (mantissa LSB / integer parity) is 0
            pick = lo if self.codes[lo] % 2 == 0 else hi
        return self._signed(pick, neg)

    def stochastic(self, y: Fraction, neg: bool, r: int) -> int:
        a = abs(y)
        if a >= self.maxnorm:
            return self._signed(len(self.values) - 1, neg)
        lo, hi = self._neighbours(a)
        if lo == hi:
            return self._signed(lo, neg)
        frac = (a - self.values[lo]) / (self.values[hi] - self.values[lo])
        F = math.floor(frac * (1 << 32))
        return self._signed(hi if r < F else lo, neg)


def floor_log2_exact(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def brute_block(grid: Grid, v, rnd=None):
    """(scale code, codes) of one block, straight from the definitions."""
    vals = [float(np.float32(x)) for x in v]
    vals = [math.copysign(0.0, x) if is_sub32(x) else x for x in vals]
    if any(not math.isfinite(x) for x in vals):
        return None
    amax = max(Fraction(abs(x)) for x in vals)
    if amax == 0:
        shared = -127
    else:
        shared = max(floor_log2_exact(amax) - grid.emax, -127)
    X = Fraction(2) ** shared
    codes = []
    for i, x in enumerate(vals):
        y = Fraction(x) / X
        neg = math.copysign(1.0, x) < 0
        if rnd is None:
            codes.append(grid.nearest_even(y, neg))
        else:
            codes.append(grid.stochastic(y, neg, int(rnd[i])))
    if grid.is_int:
        codes = [0 if c == 0 else c for c in codes]
    return shared + 127, codes
