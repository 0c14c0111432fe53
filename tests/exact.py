"""Exact-rational helpers for pinning the oracle (pure Python, small inputs).

Nothing here calls the oracle or the library.  Values of the two formats are
built from their definitions on the pages ("LongLive-2.0 ..." architecture
walkthrough, section "NVFP4 Training", paragraphs "NVFP4 numeric format" and
"Hierarchical scaling"): E2M1 has 1 sign, 2 exponent and 1 mantissa bit and
the value set {0, 0.5, 1, 1.5, 2, 3, 4, 6}; E4M3 has 4 exponent and 3 mantissa
bits with maximum 448.  The E4M3 set is enumerated here as all k * 2^j with a
3-bit fraction, independently of the oracle's bit decoding.
"""
from fractions import Fraction as Fr

import numpy as np

E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e4m3_set():
    """All finite non-negative E4M3FN values, ascending (127 values)."""
    vals = {Fr(0)}
    # subnormals: j/8 * 2^-6, j = 1..7 ; normals: (1 + j/8) * 2^e, e = -6..8
    for j in range(1, 8):
        vals.add(Fr(j, 8) * Fr(1, 64))
    for e in range(-6, 9):
        for j in range(8):
            v = (1 + Fr(j, 8)) * (Fr(2) ** e)
            if v <= 448:
                vals.add(v)
    return sorted(vals)


E4M3 = e4m3_set()


def nearest_even(a: Fr, grid):
    """Index of the nearest grid value to a (grid ascending), ties to even index;
    values beyond the last point go to the last point."""
    best, bd = 0, abs(a - grid[0])
    for i in range(1, len(grid)):
        d = abs(a - grid[i])
        if d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


def f32(x) -> Fr:
    return Fr(float(np.float32(x)))


def round_f32(v: Fr) -> Fr:
    """Round a rational to the nearest binary32 (ties to even), normal range."""
    if v == 0:
        return Fr(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fr(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return s * q * ulp


def exact_block(xs, alpha: Fr, rule4over6=True):
    """Exact-real reading of one block: returns (chosen c, scale, codes, e6, e4).

    s_c = E4M3(max|x| / (alpha c)); code = E2M1(x / (s alpha)); error is the
    exact squared X-domain reconstruction error; 4 wins only if strictly
    smaller."""
    xs = [Fr(x) for x in xs]
    m = max(abs(x) for x in xs)
    out = {}
    for c in (6, 4):
        s = E4M3[nearest_even(m / (alpha * c), E4M3)]
        codes, err = [], Fr(0)
        for x in xs:
            if s == 0:
                q = 0
            else:
                q = nearest_even(abs(x) / (s * alpha), E2M1)
            codes.append(q | (8 if x < 0 else 0))   # sign of zero is not tracked here
            err += (abs(x) - E2M1[q] * s * alpha) ** 2
        out[c] = (s, codes, err)
    c = 4 if rule4over6 and out[4][2] < out[6][2] else 6
    return c, out[c][0], out[c][1], out[6][2], out[4][2]
