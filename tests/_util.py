"""Helpers shared by the tests: fixture parsing, bf16 ulp distance, brute
force layout and exact rational rounding. None of this is used by the oracle
or by the GPU library; it is what the tests check them with."""
from __future__ import annotations

import os
from fractions import Fraction
from typing import Dict, List

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_cases(fname: str) -> List[Dict[str, List[str]]]:
    """Parse a golden text fixture: '#' comments, 'case <name>' separators,
    'key v1 v2 ...' lines."""
    cases: List[Dict[str, List[str]]] = []
    cur: Dict[str, List[str]] = {}
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                if cur:
                    cases.append(cur)
                cur = {"name": vals}
                continue
            cur[key] = vals
    if cur:
        cases.append(cur)
    return cases


def ints(v: List[str]) -> np.ndarray:
    return np.array([int(x, 0) for x in v], dtype=np.int64)


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns onto integers whose order is the numeric order
    (sign-magnitude -> two's complement); +0 and -0 both map to 0."""
    b = bits.astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a) - bf16_ordered(b))


def brute_force_layout(ids: np.ndarray, E: int, align: int = 1):
    """Quadratic-time layout straight from the definition: the row of a valid
    pair is its expert's segment start plus the number of earlier valid pairs
    (in (t, k) order) that go to the same expert."""
    N, K = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    valid = [0 <= e < E for e in flat]
    counts = [sum(1 for i, e in enumerate(flat) if valid[i] and e == x) for x in range(E)]
    offsets = [0]
    for x in range(E):
        offsets.append(offsets[-1] + -(-counts[x] // align) * align)
    pos = []
    for i, e in enumerate(flat):
        if not valid[i]:
            pos.append(-1)
            continue
        before = sum(1 for j in range(i) if valid[j] and flat[j] == e)
        pos.append(offsets[e] + before)
    bad = sum(1 for e in flat if e >= E)
    return counts, offsets, np.array(pos).reshape(N, K), bad


def round_fraction(q: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round an exact rational to the nearest binary float with ``mant_bits``
    significand bits (hidden bit included), ties to even; ``emin`` is the
    exponent of the smallest normal, ``emax`` of the largest binade.
    Returns the rounded value as a Fraction (inf as None)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    m = abs(q)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    scaled = m / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        return None
    return sign * r


def round_f32(q: Fraction) -> Fraction:
    return round_fraction(q, 24, -126, 127)


def round_bf16(q: Fraction) -> Fraction:
    return round_fraction(q, 8, -126, 127)


def f32_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def float_to_bf16_bits_exact(q: Fraction) -> int:
    """bf16 bit pattern of an exactly representable bf16 value."""
    f = np.float32(float(q))
    u = int(np.array([f], np.float32).view(np.uint32)[0])
    assert u & 0xFFFF == 0, (q, hex(u))
    return u >> 16
