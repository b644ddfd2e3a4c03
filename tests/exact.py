"""Exact-rational helpers for pinning the oracle (tests only).

These are written independently of ``oracle/``: values are Python
``Fraction``s, and rounding to float32 is done by integer arithmetic on the
rational, not by numpy.  E4M3 code values come from torch's CPU
``float8_e4m3fn`` type (a library routine), not from the oracle's decoder.
"""

from fractions import Fraction

import numpy as np
import torch

F32_MANT = 23
F32_EMIN = -126


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^(e-1) < a < 2^(e+1); fix up
    if a >= Fraction(2) ** e:
        while a >= Fraction(2) ** (e + 1):
            e += 1
    else:
        while a < Fraction(2) ** e:
            e -= 1
    return e


def round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_f32(x: Fraction) -> Fraction:
    """Nearest float32 value (ties to even), as an exact Fraction.
    No overflow handling (callers stay far below 2^128)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), F32_EMIN)
    quantum = Fraction(2) ** (e - F32_MANT)
    n = round_half_even(a / quantum)
    return sign * n * quantum


def f32_frac(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def e4m3_table() -> list:
    """Exact values of all 256 codes via torch's float8_e4m3fn (None for NaN)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    return [None if v != v else Fraction(v) for v in vals]


def nearest_code(v: Fraction, table) -> int:
    """Brute force: the finite code nearest to v; ties go to the code with an
    even mantissa (even code); zero results keep the sign of v."""
    best = None
    for c in range(256):
        t = table[c]
        if t is None:
            continue
        d = abs(t - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    c = best[1]
    if table[c] == 0:
        c = 0x80 if (v < 0) else 0x00
    return c


def nearest_code_signed(v: Fraction, negative_zero: bool, table) -> int:
    c = nearest_code(v, table)
    if v == 0 and negative_zero:
        return 0x80
    return c
