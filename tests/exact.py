"""Exact-arithmetic helpers for pinning the oracle (rationals, fp32 rounding).

Independent of the oracle: these work on ``fractions.Fraction`` values.
"""

from fractions import Fraction

import numpy as np


def exact_dot(x, w) -> Fraction:
    """The exact real dot product of two float vectors."""
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w)), Fraction(0))


def rne_f32(q: Fraction) -> np.float32:
    """Round an exact rational to fp32, nearest with ties to even (finite range)."""
    a = np.float32(float(q))
    cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - q)
        even = (int(np.array(c, dtype=np.float32).view(np.uint32)) & 1) == 0
        key = (dist, not even)
        if best is None or key < best[0]:
            best = (key, c)
    r = best[1]
    return np.float32(r) + np.float32(0.0)


def seq_error_bound(x, w) -> Fraction:
    """Bound on |sequential float64 sum - exact sum|: d * 2^-53 * sum |x_k w_k|."""
    d = len(x)
    return Fraction(d, 2 ** 53) * sum(abs(Fraction(float(a)) * Fraction(float(b)))
                                      for a, b in zip(x, w))


def near_f32_midpoint(q: Fraction, tol: Fraction) -> bool:
    """True when q lies within tol of a point where fp32 rounding changes."""
    a = np.float32(float(q))
    for c in (np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))):
        for nb in (np.nextafter(c, np.float32(np.inf)),):
            mid = (Fraction(float(c)) + Fraction(float(nb))) / 2
            if abs(q - mid) <= tol:
                return True
    return False
