"""Independent brute-force statements used to pin the CPU oracle.

Nothing here calls the oracle or the HIP library. Arithmetic is done in exact
rationals (``fractions.Fraction``) and rounded by explicit search, so a
mistake in the oracle's C code (a wrong index, a dropped term, a wrong
rounding rule) shows up as a mismatch:

* ``round_f32``   -- exact rational -> nearest fp32 (ties to even) by
  constructing the fp32 grid around the value;
* ``fma_f32``     -- w * x + acc evaluated exactly, rounded once (fused
  multiply-add semantics);
* ``E4M3_VALUES`` -- every finite float8 e4m3fn value, decoded from the bit
  layout (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  is subnormal; 0x7F / 0xFF are NaN and there is no infinity);
* ``nearest_e4m3`` -- nearest finite code by exhaustive search, ties to the
  even code, which is round-to-nearest-even with saturation at +-448;
* ``floor_log2``  -- integer floor of log2 of a positive rational by search.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def floor_log2(x: Fraction) -> int:
    """Largest integer n with 2^n <= x (x > 0), by search."""
    assert x > 0
    n = 0
    while Fraction(2) ** n > x:
        n -= 1
    while Fraction(2) ** (n + 1) <= x:
        n += 1
    return n


def round_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest fp32 value, ties to even."""
    if x == 0:
        return 0.0
    s = -1 if x < 0 else 1
    a = abs(x)
    e = floor_log2(a)
    q = Fraction(2) ** (max(e, -126) - 23)   # grid spacing (subnormal below 2^-126)
    n = a / q
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * q
    if v >= Fraction(2) ** 128:
        return s * math.inf
    return s * float(v)   # exact: an fp32 value is a double


def fma_f32(w: float, x: float, acc: float) -> float:
    return round_f32(Fraction(w) * Fraction(x) + Fraction(acc))


def add_f32(a: float, b: float) -> float:
    return round_f32(Fraction(a) + Fraction(b))


def brute_routed_sum(payload_f, src_info, weights, shared_f=None):
    """Routed fp32 sum for tiny shapes: payload_f [ep, mtpr, H] float values,
    weights [T, k] or None, shared_f [T, H] or None. Returns [T][H] floats."""
    T, k, _ = src_info.shape
    H = payload_f.shape[2]
    out = []
    for t in range(T):
        row = []
        for h in range(H):
            acc = 0.0
            for j in range(k):
                r, rr = int(src_info[t, j, 0]), int(src_info[t, j, 1])
                if r < 0:
                    continue
                w = 1.0 if weights is None else float(weights[t, j])
                acc = fma_f32(w, float(payload_f[r, rr, h]), acc)
            if shared_f is not None:
                acc = add_f32(acc, float(shared_f[t, h]))
            row.append(acc)
        out.append(row)
    return out


def _e4m3_decode(code: int) -> Fraction:
    s = -1 if code & 0x80 else 1
    E = (code >> 3) & 0xF
    m = code & 0x7
    if E == 0:
        v = Fraction(m, 8) * Fraction(2) ** -6
    else:
        v = (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7)
    return s * v


# finite non-negative codes 0x00..0x7E and their values
E4M3_CODES = list(range(0x7F))
E4M3_VALUES = [_e4m3_decode(c) for c in E4M3_CODES]
E4M3_FLOATS = np.array([float(v) for v in E4M3_VALUES], dtype=np.float64)


def e4m3_decode(code: int) -> float:
    return float(_e4m3_decode(code))


def nearest_e4m3(q: float) -> int:
    """Nearest finite e4m3 code (ties -> even code), sign from q."""
    a = Fraction(abs(q)) if math.isfinite(q) else Fraction(10 ** 6)
    best, bd = None, None
    for c, v in zip(E4M3_CODES, E4M3_VALUES):
        d = abs(a - v)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    neg = math.copysign(1.0, q) < 0
    return best | (0x80 if neg else 0)


def nearest_e4m3_vec(q: np.ndarray) -> np.ndarray:
    """Vectorised ``nearest_e4m3`` for finite float64 inputs (exact: every
    fp32 value and every e4m3 value is a double, and the distances compared
    here are differences of doubles that are exact for these magnitudes
    because both operands lie on a common 2^-149 grid within 2^10)."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), 1024.0)
    d = np.abs(a[:, None] - E4M3_FLOATS[None, :])
    dmin = d.min(axis=1, keepdims=True)
    tie = d == dmin
    codes = np.arange(0x7F)
    # among the tied candidates prefer the even code
    even_tie = tie & (codes[None, :] % 2 == 0)
    pick = np.where(even_tie.any(axis=1), even_tie.argmax(axis=1), tie.argmax(axis=1))
    neg = np.signbit(q)
    return (pick | np.where(neg, 0x80, 0)).astype(np.uint8)
