"""Pins of the oracle's element and scale formats (CPU only).

E2M1 and E4M3 are checked against exact-rational nearest searches over value
sets built from their definitions (tests/exact.py), against the golden value
table, and E4M3 additionally against torch's float8_e4m3fn conversion (a
library routine with the same rounding for |t| <= 448)."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.exact import E2M1, E4M3, Fr, nearest_even

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    out = {}
    for line in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        out[int(code, 16)] = val
    return out


def test_e2m1_decode_table_matches_pages():
    g = _golden_e2m1()
    assert len(g) == 16
    for code, val in g.items():
        v = oracle.e2m1_value(code)
        assert v == float(val)
        assert np.signbit(v) == val.startswith("-")


def test_e2m1_encode_ties_and_saturation():
    # ties go to the even code; anything at or beyond 6 saturates to 6
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             6.0: 7, 6.5: 7, 100.0: 7, 3e38: 7, 0.0: 0, 1e-45: 0}
    for v, code in table.items():
        assert oracle.e2m1_encode(v) == code, v
        assert oracle.e2m1_encode(-v) == code | 8, -v
    assert oracle.e2m1_encode(-0.0) == 8


def _probe_values(grid, rng, n_random, hi):
    vals = []
    pts = [float(g) for g in grid]
    mids = [float((grid[i] + grid[i + 1]) / 2) for i in range(len(grid) - 1)]
    for p in pts + mids:
        f = np.float32(p)
        vals += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    vals += list(rng.uniform(0, hi, n_random).astype(np.float32))
    return [v for v in vals if v >= 0]


def test_e2m1_encode_matches_exact_nearest():
    rng = np.random.default_rng(11)
    for v in _probe_values(E2M1, rng, 3000, 8.0):
        want = nearest_even(Fr(float(v)), E2M1)
        assert oracle.e2m1_encode(float(v)) == want, v
        assert oracle.e2m1_encode(-float(v)) == (want | 8), v


def test_e4m3_value_set():
    vals = [oracle.e4m3_value(b) for b in range(127)]
    assert [Fr(v) for v in vals] == E4M3            # ascending, same set
    assert len(E4M3) == 127
    assert max(vals) == 448.0                        # M_FP8
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    # library cross-check of the bit layout
    t = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(t, np.array(vals, np.float32))


def test_e4m3_encode_matches_exact_nearest_and_torch():
    rng = np.random.default_rng(12)
    vals = _probe_values(E4M3, rng, 4000, 460.0)
    for v in vals:
        want = nearest_even(Fr(float(v)), E4M3)
        assert oracle.e4m3_encode(float(v)) == want, v
    small = np.array([v for v in vals if v <= 448.0], np.float32)
    tb = torch.from_numpy(small).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in small], np.uint8)
    assert np.array_equal(got, tb)


def test_e4m3_saturates_instead_of_nan():
    for t in (448.0, 460.0, 464.0, 464.001, 480.0, 672.0, 1e6, 3e38):
        assert oracle.e4m3_encode(t) == 126, t
    # below half the smallest subnormal rounds to zero; exactly half ties to 0
    assert oracle.e4m3_encode(2.0 ** -10) == 0
    assert oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1
    assert oracle.e4m3_encode(1.5 * 2.0 ** -9) == 2          # tie 1 vs 2 -> even


def test_global_scale_reading():
    # alpha = amax / (448 * 6); zero tensor -> 1
    assert oracle.global_scale(2688.0) == 1.0
    for k in (-20, -3, 0, 7, 30):
        assert oracle.global_scale(2688.0 * 2.0 ** k) == np.float32(2.0 ** k)
    assert oracle.global_scale(0.0) == 1.0
    a = np.float32(3.7)
    assert oracle.global_scale(a) == np.float32(a / np.float32(2688.0))


def test_constants_golden():
    c = {}
    for line in open(os.path.join(GOLDEN, "format_constants.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        c[k] = float(v)
    assert oracle.e4m3_value(126) == c["m_fp8"]
    assert oracle.e2m1_value(7) == c["m_fp4"]
    assert oracle.global_scale(c["m_fp8"] * c["m_fp4"]) == 1.0
    assert c["bytes_per_elem"] == 0.5 + 1.0 / c["block_elems"]
    assert abs(4.0 / (2 * c["bytes_per_elem"]) - c["kv_compression"]) < 1e-12
