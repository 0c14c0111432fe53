"""Tie-driving NVFP4 test tensors (inputs only; no method arithmetic).

Every tensor holds one element equal to 2688 = 448 * 6, so alpha = 1 exactly.
e2m1_tie_tensor: blocks with maximum 6 * 2^j, so the block scale is 2^j and
its reciprocal exact; the other elements are E2M1 midpoints times 2^j and one
unit in the last place either side, both signs, with the codes that
round-to-nearest-even gives them (a closed form: below a midpoint the lower
code, above it the upper, at it the even one).
e4m3_tie_tensor: blocks whose max / 6 (rule 0) or max / 4 (rule 1) is an E4M3
midpoint, one ulp either side, 2^-9, or in the saturating zone 448 ... 672.
"""
import numpy as np

import workloads
from tests.exact import E4M3, Fr

MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
LOWER = {0.25: 0, 0.75: 1, 1.25: 2, 1.75: 3, 2.5: 4, 3.5: 5, 5.0: 6}     # E2M1 code just below the midpoint
JS = range(-9, 9)                                                       # s = 2^j, every power of two E4M3 holds


def step_ulps(v: np.ndarray, d: int, bf16: bool) -> np.ndarray:
    """v moved by d units in the last place (of fp32, or of bf16) away from
    zero (d > 0) or toward it (d < 0); v > 0."""
    if d == 0:
        return v
    if bf16:
        b = workloads.f32_to_bf16_bits(v.astype(np.float32)).astype(np.int64) + d
        return workloads.bf16_to_f32(b.astype(np.uint16)).astype(np.float32)
    return np.nextafter(v.astype(np.float32), np.float32(np.inf if d > 0 else 0)).astype(np.float32)


def _e4m3_byte_of_pow2(j: int) -> int:
    return (j + 7) << 3 if j >= -6 else 1 << (j + 9)


def e2m1_tie_tensor(bf16: bool):
    """(x [rows, 16] fp32 values, expected STATIC6 codes [rows, 16], expected
    scale bytes [rows]); row 0 holds 2688."""
    rows, codes, sbytes = [], [], []
    x0 = np.zeros(16, np.float32)
    x0[0] = 2688.0
    rows.append(x0)
    codes.append(None)
    sbytes.append(None)
    for j in JS:
        vals, want = [], []
        for v in MIDS:
            base = np.float32(v * 2.0 ** j)
            for d in (-1, 0, 1):
                mag = step_ulps(np.array([base]), d, bf16)[0]
                code = LOWER[v] + (1 if d > 0 else 0) + (1 if d == 0 and LOWER[v] % 2 == 1 else 0)
                for sign in (1.0, -1.0):
                    vals.append(sign * mag)
                    want.append(code | (8 if sign < 0 else 0))
        for c0 in range(0, len(vals), 15):
            blk = np.zeros(16, np.float32)
            wc = np.zeros(16, np.int64)
            blk[0] = np.float32(6.0 * 2.0 ** j)
            wc[0] = 7
            part = vals[c0:c0 + 15]
            blk[1:1 + len(part)] = part
            wc[1:1 + len(part)] = want[c0:c0 + 15]
            rows.append(blk)
            codes.append(wc)
            sbytes.append(_e4m3_byte_of_pow2(j))
    return np.stack(rows), codes, sbytes


def unpack_codes(c: np.ndarray) -> np.ndarray:
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)


def to_input(x: np.ndarray, bf16: bool):
    if bf16:
        bits = workloads.f32_to_bf16_bits(x)
        assert np.array_equal(workloads.bf16_to_f32(bits), x)     # every value is a bf16 value
        return bits
    return x


def _e4m3_targets():
    """Every midpoint between consecutive non-negative E4M3 values (2^-10 ...
    432), the E4M3 values 2^-9 and 448, and the saturating zone 448 ... 672
    (reachable by max/4 only: max <= 2688)."""
    mids = [(E4M3[i] + E4M3[i + 1]) / 2 for i in range(len(E4M3) - 1)]
    extra = [E4M3[1], Fr(448), Fr(456), Fr(464), Fr(500), Fr(600), Fr(672)]
    return [float(t) for t in mids + extra]


def _block_of_max(m: np.float32, g: np.random.Generator) -> np.ndarray:
    blk = (g.uniform(-1, 1, 16) * m).astype(np.float32)
    blk[0] = m
    blk[5] = np.float32(-m)
    return blk


def e4m3_tie_tensor(rule: int):
    """(x fp32 [rows, 16], the scale target max/c of each row or None).
    STATIC6: max = m with fp32(m / 6) == target; 4OVER6: max = 4 * target."""
    g = np.random.default_rng(7)
    rows, targets = [], []
    x0 = np.zeros(16, np.float32)
    x0[0] = 2688.0
    rows.append(x0)
    targets.append(None)
    for t in _e4m3_targets():
        for d in (-1, 0, 1):
            tt = step_ulps(np.array([t], np.float32), d, False)[0]
            if rule == 1:
                m = np.float32(4.0) * tt
                if m > 2688.0:
                    continue
            else:
                if tt > 448.0:
                    continue
                m = None
                c = np.float32(6.0) * tt
                for k in range(-4, 5):                      # fp32 neighbours of 6 t
                    cand = c
                    for _ in range(abs(k)):
                        cand = np.nextafter(cand, np.float32(np.inf if k > 0 else 0))
                    if np.float32(cand / np.float32(6.0)) == tt and cand <= 2688.0:
                        m = np.float32(cand)
                        break
                if m is None:
                    continue
            rows.append(_block_of_max(m, g))
            targets.append(tt)
    return np.stack(rows), targets
