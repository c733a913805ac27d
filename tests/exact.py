"""Exact-arithmetic helpers for pinning the oracle.

``round_f32`` rounds an exact rational to the nearest float32 (ties to even,
subnormals kept, overflow to infinity) using only integer arithmetic, so a
float32 expression can be evaluated step by step without relying on any
floating-point unit. Used to check the oracle's squared distance bit for bit.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_EMIN = -126          # smallest normal exponent of float32
_MANT = 23            # stored mantissa bits
_MAX = Fraction((1 << 24) - 1, 1) * Fraction(2) ** (127 - 23)


def round_f32(x: Fraction) -> Fraction:
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # e = floor(log2(a))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, _EMIN) - _MANT)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r > _MAX:
        return Fraction(sign) * Fraction(10) ** 400  # stands for infinity
    return sign * r


def to_f32(x: Fraction) -> np.float32:
    if abs(x) > _MAX:
        return np.float32(np.inf) * (1 if x > 0 else -1)
    # x is a float32 value, exactly representable in float64
    return np.float32(float(x))


def s32_exact(a, b) -> np.float32:
    """((dx*dx + dy*dy) + dz*dz) with every operation rounded to float32."""
    A = [Fraction(float(np.float32(v))) for v in a]
    B = [Fraction(float(np.float32(v))) for v in b]
    d = [round_f32(A[i] - B[i]) for i in range(3)]
    sq = [round_f32(di * di) for di in d]
    return to_f32(round_f32(round_f32(sq[0] + sq[1]) + sq[2]))


def s32_exact_alternatives(a, b) -> dict:
    """The same distance under orders the pages rule out, to show a test can
    tell them apart: right-to-left sum, fused multiply-add accumulation, and a
    single rounding of the exact result."""
    A = [Fraction(float(np.float32(v))) for v in a]
    B = [Fraction(float(np.float32(v))) for v in b]
    d = [round_f32(A[i] - B[i]) for i in range(3)]
    sq = [round_f32(di * di) for di in d]
    right = round_f32(sq[0] + round_f32(sq[1] + sq[2]))
    fma = round_f32(d[2] * d[2] + round_f32(d[1] * d[1] + round_f32(d[0] * d[0])))
    exact = round_f32(sum((A[i] - B[i]) ** 2 for i in range(3)))
    return {"right_to_left": to_f32(right), "fma_chain": to_f32(fma), "one_rounding": to_f32(exact)}


def f32_bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])
