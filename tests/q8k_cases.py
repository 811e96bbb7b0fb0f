"""Test helper: activation chunks that pin down how the Q8_K code is formed,
and the code's definition in exact rational arithmetic.

The Q8_K form (K-quant kernel arc page, "The pieces", kq v2 item) scales
each 256-value chunk by d8 = amax/127 and codes every value as the nearest
integer to x/d8.  The reading taken here: both divisions are IEEE binary32
divisions (correctly rounded, ties to even) and the code is the binary32
quotient rounded half to even.  A reciprocal multiply x * (1/d8) is not the
same function: for some x it lands on the other side of a .5 boundary.
Random N(0,1) rows almost never show that, so these chunks are built to sit
exactly where the two disagree.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32


def round_binary32(v: Fraction) -> Fraction:
    """The binary32 value nearest to v (ties to even), normal range only."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    assert -126 <= e <= 127, "outside the normal binary32 range"
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def round_half_even(v: Fraction) -> int:
    n = v.numerator // v.denominator  # floor
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def exact_q8k_chunk(x: np.ndarray):
    """Codes and scale of one 256-value chunk by the definition, in exact
    rationals: d8 = binary32(amax/127), code = rint(binary32(x/d8)) clamped
    to [-127, 127]; an all-zero chunk gives d8 = 0 and zero codes."""
    x = np.asarray(x, F32)
    assert x.shape == (256,)
    amax = max(Fraction(float(abs(v))) for v in x)
    if amax == 0:
        return np.zeros(256, np.int64), Fraction(0)
    d8 = round_binary32(amax / 127)
    codes = [max(-127, min(127, round_half_even(round_binary32(Fraction(float(v)) / d8)))) for v in x]
    return np.asarray(codes, np.int64), d8


def reciprocal_codes(x: np.ndarray) -> np.ndarray:
    """The rejected reading (binary32 x * (1/d8)), for showing that the chunks
    tell the two apart."""
    x = np.asarray(x, F32)
    d8 = np.abs(x).max() / F32(127)
    r = F32(1) / d8
    return np.clip(np.rint(x * r), -127, 127).astype(np.int64)


def quotient_chunks(count: int, seed: int, per_chunk: int = 24) -> np.ndarray:
    """`count` chunks of 256 float32 values: value 0 is the chunk's amax, and
    `per_chunk` values sit next to a .5 boundary of x/d8 where the binary32
    quotient and the binary32 reciprocal product round to different codes;
    the rest are N(0,1) draws scaled below amax.  Found by a seeded search
    (numpy float32 arithmetic only chooses candidates; what a chunk must give
    is fixed by exact_q8k_chunk)."""
    rng = np.random.default_rng(seed)
    out = np.empty((count, 256), F32)
    for c in range(count):
        while True:
            amax = F32(rng.uniform(0.25, 6.0)) * F32(2.0 ** int(rng.integers(-6, 6)))
            d8 = amax / F32(127)
            r = F32(1) / d8
            found = []
            for _ in range(4000):
                k = int(rng.integers(-126, 126))
                base = F32((k + 0.5) * float(d8))
                for step in range(-3, 4):
                    v = base
                    for _ in range(abs(step)):
                        v = np.nextafter(v, F32(np.inf) if step > 0 else F32(-np.inf))
                    if abs(v) < amax and np.rint(v / d8) != np.rint(v * r):
                        found.append(v)
                if len(found) >= per_chunk:
                    break
            if len(found) >= per_chunk:
                break
        chunk = (rng.standard_normal(256).astype(F32) * (amax / F32(5))).clip(-amax * F32(0.99), amax * F32(0.99))
        chunk[0] = amax if rng.integers(0, 2) else -amax
        pos = rng.choice(np.arange(1, 256), size=per_chunk, replace=False)
        chunk[pos] = np.asarray(found[:per_chunk], F32)
        out[c] = chunk
    return out
