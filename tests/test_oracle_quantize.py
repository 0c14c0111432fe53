"""Pins of the oracle quantizer (CPU only).

What fixes each expected value:
  * the worked four-over-six example (golden file, derived from the pages);
  * exact round trips of blocks built from representable values;
  * zero blocks / zero tensors;
  * invariants of the rule (power-of-two scaling, sign symmetry, geometry
    identities, static-6 inside four-over-six, error bounds);
  * an exact-rational re-derivation of both candidates (tests/exact.py) on
    random and small-alphabet blocks: every disagreement must be a near tie
    of the real-valued rule (the fp32 evaluation order is a reading).
"""
import os

import numpy as np
import pytest

import oracle
from oracle import COL16, FOUR_OVER_SIX, ROW16, STATIC6, TILE16
from tests.exact import E2M1, E4M3, Fr, exact_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_F = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def unpack(codes: np.ndarray) -> np.ndarray:
    """[r, c/2] bytes -> [r, c] nibbles (element 2j = low nibble)."""
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def code_values(nib):
    v = E2M1_F[nib & 7]
    return np.where(nib & 8, -v, v)


def e4m3_f(b):
    return np.array([oracle.e4m3_value(int(v)) for v in np.asarray(b).ravel()]).reshape(np.shape(b))


# ------------------------------------------------------------- worked example

def test_four_over_six_worked_example():
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1] = 6.0, 4.5
    x[0, 16] = 2688.0
    rows = [l.split() for l in open(os.path.join(GOLDEN, "four_over_six_example.txt"))
            if l.strip() and not l.startswith("#")]
    for rule_name, blk, sb, codes, deq in rows:
        rule = FOUR_OVER_SIX if rule_name == "4over6" else STATIC6
        p = oracle.quantize(x, ROW16, rule)
        blk = int(blk)
        assert p.alpha == 1.0
        assert p.scales[0, blk] == int(sb, 16)
        nib = unpack(p.codes)[0, blk * 16:(blk + 1) * 16]
        assert list(nib) == [int(c) for c in codes.split(",")]
        y = oracle.dequantize(p)
        assert list(y[0, blk * 16: blk * 16 + 2]) == [float(v) for v in deq.split(",")]
    # the 4-candidate was chosen exactly once (block 0)
    assert oracle.quantize(x, ROW16, FOUR_OVER_SIX).stats[0] == 1


# ------------------------------------------------------------- round trips

def _representable(rng, rows, cols, block, k):
    """x = q * s * 2^k with one element equal to 2688 * 2^k (so alpha = 2^k)
    and each block's max equal to 6 * s (so the 6-candidate is exact)."""
    x = np.zeros((rows, cols), np.float64)
    if block == ROW16:
        groups = [(r, slice(c, c + 16)) for r in range(rows) for c in range(0, cols, 16)]
    elif block == TILE16:
        groups = [(slice(r, r + 16), slice(c, c + 16)) for r in range(0, rows, 16) for c in range(0, cols, 16)]
    else:
        groups = [(slice(r, r + 16), c) for c in range(cols) for r in range(0, rows, 16)]
    for gi, (gr, gc) in enumerate(groups):
        # normal E4M3 scale; the first block holds 2688 = 6 * 448, so s = 448
        sb = 126 if gi == 0 else int(rng.integers(8, 127))
        s = oracle.e4m3_value(sb)
        blk = x[gr, gc]
        q = E2M1_F[rng.integers(0, 8, size=blk.shape)] * np.where(rng.random(blk.shape) < 0.5, -1, 1)
        flat = q.reshape(-1)
        flat[rng.integers(0, flat.size)] = 6.0 * (1 if rng.random() < 0.5 else -1)
        x[gr, gc] = q * s
    x[0, 0] = 2688.0          # alpha = 1 before scaling; block 0 has max 6 * 448
    return (x * 2.0 ** k).astype(np.float32)


@pytest.mark.parametrize("block", [ROW16, TILE16, COL16])
@pytest.mark.parametrize("rule", [STATIC6, FOUR_OVER_SIX])
@pytest.mark.parametrize("k", [-7, 0, 5])
def test_exact_round_trip(block, rule, k):
    rng = np.random.default_rng(100 + block * 10 + rule + k)
    x = _representable(rng, 32, 64, block, k)
    p = oracle.quantize(x, block, rule)
    assert p.alpha == np.float32(2.0 ** k)
    y = oracle.dequantize(p)
    assert np.array_equal(y, x)
    if rule == FOUR_OVER_SIX:
        assert p.stats[0] == 0          # e6 == 0 everywhere: ties keep 6


# ------------------------------------------------------------- zero cases

@pytest.mark.parametrize("block", [ROW16, TILE16, COL16])
def test_zero_tensor(block):
    x = np.zeros((16, 32), np.float32)
    x[3, 5] = -0.0
    x[7, ::3] = -0.0
    p = oracle.quantize(x, block, FOUR_OVER_SIX)
    assert p.alpha == 1.0
    assert not p.scales.any()
    y = oracle.dequantize(p)
    assert np.array_equal(np.signbit(y), np.signbit(x)) and not y.any()


def test_zero_block_inside_tensor():
    x = np.zeros((2, 32), np.float32)
    x[0, :16] = np.linspace(-3, 3, 16)
    x[1, 16:] = -0.0
    p = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    assert p.scales[0, 1] == 0 and p.scales[1, 0] == 0 and p.scales[1, 1] == 0
    nib = unpack(p.codes)
    assert (nib[1, 16:] == 8).all() and (nib[1, :16] == 0).all()


# ------------------------------------------------------------- invariants

def _rand(seed, shape, sigma=1.0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * sigma
    if outliers:
        idx = rng.choice(x.size, size=max(1, x.size // 500), replace=False)
        x.reshape(-1)[idx] *= 50
    return x.astype(np.float32)


@pytest.mark.parametrize("block", [ROW16, TILE16, COL16])
def test_power_of_two_scaling_invariance(block):
    x = _rand(1, (48, 64))
    p = oracle.quantize(x, block, FOUR_OVER_SIX)
    for k in (-9, -1, 3, 11):
        q = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32), block, FOUR_OVER_SIX)
        assert np.array_equal(q.codes, p.codes) and np.array_equal(q.scales, p.scales)
        assert q.alpha == np.float32(p.alpha * 2.0 ** k)


@pytest.mark.parametrize("block", [ROW16, TILE16, COL16])
def test_sign_symmetry(block):
    x = _rand(2, (32, 48))
    x[0, :5] = 0.0
    p = oracle.quantize(x, block, FOUR_OVER_SIX)
    q = oracle.quantize(-x, block, FOUR_OVER_SIX)
    assert np.array_equal(q.scales, p.scales) and q.alpha == p.alpha
    assert np.array_equal(q.codes, p.codes ^ 0x88)


def test_col16_is_row16_of_transpose():
    x = _rand(3, (64, 48))
    c = oracle.quantize(x, COL16, FOUR_OVER_SIX)
    r = oracle.quantize(np.ascontiguousarray(x.T), ROW16, FOUR_OVER_SIX)
    assert np.array_equal(c.codes, r.codes) and np.array_equal(c.scales, r.scales) and c.alpha == r.alpha
    assert np.array_equal(oracle.dequantize(c), oracle.dequantize(r).T)


def test_tile16_single_row_equals_row16():
    # a 16x16 tile with one non-zero row: the other rows add zero error and
    # cannot change the block max, so the tile quantizes like that row's 1D block
    rng = np.random.default_rng(4)
    x = np.zeros((16, 64), np.float32)
    x[5] = rng.standard_normal(64).astype(np.float32)
    x[5, 0] = 9.0
    t = oracle.quantize(x, TILE16, FOUR_OVER_SIX)
    r = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    assert np.array_equal(t.scales[0], r.scales[5])
    assert np.array_equal(t.codes, r.codes)


def test_static6_is_subset_of_four_over_six():
    x = _rand(5, (64, 256))
    s6 = oracle.quantize(x, ROW16, STATIC6)
    fo = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    same = np.repeat(s6.scales == fo.scales, 8, axis=1)
    # where the scale is unchanged the codes are unchanged
    assert np.array_equal(s6.codes[same], fo.codes[same])
    # the 4-candidate scale is E4M3(mu/4) >= the 6-candidate scale
    changed = s6.scales != fo.scales
    assert (fo.scales[changed] >= s6.scales[changed]).all()
    # a block that picks 4 always changes its scale byte (equal bytes give
    # equal codes, equal errors, and the tie keeps 6)
    assert fo.stats[0] == int(changed.sum())


def _block_sse(x, y, block_rows, block_cols):
    d = (x.astype(np.float64) - y.astype(np.float64)) ** 2
    r, c = d.shape
    return d.reshape(r // block_rows, block_rows, c // block_cols, block_cols).sum(axis=(1, 3))


@pytest.mark.parametrize("block", [ROW16, TILE16])
def test_chosen_error_not_larger(block):
    x = _rand(6, (64, 128))
    fo = oracle.quantize(x, block, FOUR_OVER_SIX)
    s6 = oracle.quantize(x, block, STATIC6)
    br = 16 if block == TILE16 else 1
    e_fo = _block_sse(x, oracle.dequantize(fo), br, 16)
    e_s6 = _block_sse(x, oracle.dequantize(s6), br, 16)
    # fp64 re-evaluation of the fp32 chain: allow a relative 1e-5 near tie
    assert (e_fo <= e_s6 * (1 + 1e-5) + 1e-30).all()
    assert (e_fo < e_s6).sum() > 0          # the rule does something on this data


def test_elementwise_error_bound():
    x = _rand(7, (64, 128))
    p = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    y = oracle.dequantize(p).astype(np.float64)
    s = e4m3_f(p.scales).repeat(16, axis=1) * float(p.alpha)
    nib = unpack(p.codes)
    q = np.abs(code_values(nib))
    # half the distance to the neighbouring grid values around q
    grid = E2M1_F
    idx = (nib & 7).astype(np.int64)
    up = np.where(idx < 7, grid[np.minimum(idx + 1, 7)] - grid[idx], 0.0)
    dn = np.where(idx > 0, grid[idx] - grid[np.maximum(idx - 1, 0)], 0.5)
    half = np.maximum(up, dn) / 2
    v = np.abs(x.astype(np.float64)) / np.where(s > 0, s, 1)
    sat = v > 6
    err = np.abs(x - y)
    bound = np.where(sat, (v - 6) * s, half * s) * (1 + 1e-5) + np.abs(x) * 2e-7
    bound = np.where(s == 0, np.abs(x), bound)
    assert (err <= bound + 1e-30).all()


def test_byte_counts():
    x = _rand(8, (32, 256))
    p = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    assert p.codes.nbytes + p.scales.nbytes == x.size * 0.5625
    t = oracle.quantize(x, TILE16, FOUR_OVER_SIX)
    assert t.scales.size == x.size // 256


# ------------------------------------------------- exact-rational brute force

def _near_tie(xs, alpha, m):
    """True if the real-valued rule is within fp32 rounding of a decision
    boundary for this block (E4M3 midpoint, E2M1 midpoint or e4 == e6)."""
    a = Fr(float(alpha))
    c, s, codes, e6, e4 = exact_block(xs, a)
    if e6 == e4 or (max(e6, e4) > 0 and abs(e6 - e4) / max(e6, e4) < Fr(1, 10 ** 5)):
        return True
    for cand in (6, 4):
        t = Fr(float(m)) / (a * cand)
        for i in range(len(E4M3) - 1):
            mid = (E4M3[i] + E4M3[i + 1]) / 2
            if mid > 0 and abs(t - mid) / mid < Fr(1, 10 ** 6):
                return True
        sc = E4M3[min(range(len(E4M3)), key=lambda i: (abs(t - E4M3[i]), i % 2))]
        if sc == 0:
            continue
        for x in xs:
            v = abs(Fr(float(x))) / (sc * a)
            for i in range(7):
                mid = (E2M1[i] + E2M1[i + 1]) / 2
                if abs(v - mid) / mid < Fr(1, 10 ** 6):
                    return True
    return False


def _compare_exact(x, rule=FOUR_OVER_SIX, block=ROW16):
    """Every block of x (ROW16: 16 along a row; TILE16: a 16x16 tile in
    row-major order) against the exact-rational rule: (disagreements that are
    not near ties, near-tie disagreements)."""
    p = oracle.quantize(x, block, rule)
    nib = unpack(p.codes)
    alpha = Fr(float(p.alpha))
    bad, ties = 0, 0
    if block == ROW16:
        blocks = [((r, b), (slice(r, r + 1), slice(b * 16, (b + 1) * 16)))
                  for r in range(x.shape[0]) for b in range(x.shape[1] // 16)]
    else:
        blocks = [((rb, cb), (slice(rb * 16, (rb + 1) * 16), slice(cb * 16, (cb + 1) * 16)))
                  for rb in range(x.shape[0] // 16) for cb in range(x.shape[1] // 16)]
    for sidx, sl in blocks:
        xs = [float(v) for v in x[sl].ravel()]
        c, s, codes, e6, e4 = exact_block(xs, alpha, rule == FOUR_OVER_SIX)
        got_s = Fr(oracle.e4m3_value(int(p.scales[sidx])))
        got_c = [int(v) & 7 for v in nib[sl].ravel()]
        want_c = [v & 7 for v in codes]
        if got_s != s or got_c != want_c:
            m = max(abs(v) for v in xs)
            if _near_tie(xs, alpha, m):
                ties += 1
            else:
                bad += 1
    return bad, ties


def test_exact_rational_random_blocks():
    x = _rand(9, (24, 256))
    bad, ties = _compare_exact(x)
    assert bad == 0
    assert ties <= 2


def test_exact_rational_small_alphabet_blocks():
    # values on a coarse dyadic grid hit many exact ties of the real-valued
    # rule; disagreements must all be such ties
    rng = np.random.default_rng(10)
    alphabet = np.arange(0, 49) / 8.0
    x = rng.choice(alphabet, size=(16, 256)) * np.where(rng.random((16, 256)) < 0.5, -1, 1)
    x[0, 0] = 2688.0
    x = x.astype(np.float32)
    bad, ties = _compare_exact(x)
    assert bad == 0


def test_exact_rational_two_value_family():
    # block {6, y, 0...} with alpha = 1: sweep y over (0, 6]; the exact rule
    # picks 4 exactly when y's error under s=1.5 is smaller than under s=1
    ys = np.unique(np.concatenate([np.linspace(0.01, 6, 241), np.arange(1, 49) / 8.0])).astype(np.float32)
    x = np.zeros((len(ys) + 1, 16), np.float32)
    x[:-1, 0] = 6.0
    x[:-1, 1] = ys
    x[-1, 0] = 2688.0
    p = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    assert p.alpha == 1.0
    for i, y in enumerate(ys):
        yy = Fr(float(y))
        e6 = (yy - E2M1[min(range(8), key=lambda j: (abs(yy - E2M1[j]), j % 2))]) ** 2
        v4 = yy / Fr(3, 2)
        e4 = (yy - Fr(3, 2) * E2M1[min(range(8), key=lambda j: (abs(v4 - E2M1[j]), j % 2))]) ** 2
        want = 0x3C if e4 < e6 else 0x38
        got = int(p.scales[i, 0])
        if got != want:
            # only where the exact comparison is a tie, or y/1.5 is an E2M1
            # midpoint that the fp32 reciprocal lands on the other side of
            mids = [(E2M1[j] + E2M1[j + 1]) / 2 for j in range(7)]
            assert e4 == e6 or v4 in mids, (float(y), got, want)


def test_exact_rational_tile16_random_tiles():
    # 16x16 weight tiles: one scale per 256 elements, the 6-vs-4 choice on the
    # whole tile's squared error (NVFP4 training recipe: 2D weight blocks)
    x = _rand(19, (64, 256), sigma=0.02)
    bad, ties = _compare_exact(x, FOUR_OVER_SIX, TILE16)
    assert bad == 0
    assert ties <= 2
    bad, ties = _compare_exact(x, STATIC6, TILE16)
    assert bad == 0


def test_exact_rational_tile16_small_alphabet_tiles():
    rng = np.random.default_rng(20)
    alphabet = np.arange(0, 49) / 8.0
    x = rng.choice(alphabet, size=(48, 128)) * np.where(rng.random((48, 128)) < 0.5, -1, 1)
    # per-tile magnitudes spread over many E4M3 binades
    x = x * (2.0 ** rng.integers(-8, 6, (3, 8))).repeat(16, axis=0).repeat(16, axis=1)
    x[0, 0] = 2688.0
    x = x.astype(np.float32)
    bad, ties = _compare_exact(x, FOUR_OVER_SIX, TILE16)
    assert bad == 0


def test_exact_rational_tile16_two_value_family():
    # tile {6 at (0, 0), y at (7, 9), 0 elsewhere} with alpha = 1: the tile's
    # squared error is that of the two values, so the exact rule picks the
    # 4-candidate (scale 1.5, byte 0x3C) iff y's error under 1.5 is smaller
    ys = np.unique(np.concatenate([np.linspace(0.01, 6, 97), np.arange(1, 49) / 8.0])).astype(np.float32)
    x = np.zeros((16, 16 * (len(ys) + 1)), np.float32)
    for i, y in enumerate(ys):
        x[0, 16 * i] = 6.0
        x[7, 16 * i + 9] = y
    x[3, -1] = 2688.0
    p = oracle.quantize(x, TILE16, FOUR_OVER_SIX)
    assert p.alpha == 1.0
    mids = [(E2M1[j] + E2M1[j + 1]) / 2 for j in range(7)]
    for i, y in enumerate(ys):
        yy = Fr(float(y))
        e6 = (yy - E2M1[min(range(8), key=lambda j: (abs(yy - E2M1[j]), j % 2))]) ** 2
        v4 = yy / Fr(3, 2)
        e4 = (yy - Fr(3, 2) * E2M1[min(range(8), key=lambda j: (abs(v4 - E2M1[j]), j % 2))]) ** 2
        want = 0x3C if e4 < e6 else 0x38
        got = int(p.scales[0, i])
        if got != want:
            assert e4 == e6 or v4 in mids, (float(y), got, want)
    # the same pairs as 1x16 blocks decide the same way (the zeros add no error)
    r = np.zeros((len(ys), 16), np.float32)
    r[:, 0] = 6.0
    r[:, 9] = ys
    r = np.concatenate([r, np.full((1, 16), 0, np.float32)])
    r[-1, 0] = 2688.0
    q = oracle.quantize(r, ROW16, FOUR_OVER_SIX)
    assert np.array_equal(q.scales[:-1, 0], p.scales[0, :-1])


def test_exact_reading_diagnostic_rate():
    # the C diagnostic (exact-real reading) vs the fp32 reading on a
    # DiT-like activation tensor: codes differ only at near ties
    x = _rand(11, (256, 1024))
    a = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    b = oracle.quantize_exact_reading(x, ROW16, FOUR_OVER_SIX)
    assert a.alpha == b.alpha
    diff_blocks = (unpack(a.codes) != unpack(b.codes)).reshape(256, 64, 16).any(axis=2) | (a.scales != b.scales)
    assert diff_blocks.mean() < 1e-3
    # and the C diagnostic itself agrees with the Python exact re-derivation
    xs = x[:4, :256]
    c = oracle.quantize_exact_reading(np.ascontiguousarray(xs), ROW16, FOUR_OVER_SIX)
    alpha = Fr(float(c.alpha))
    for r in range(4):
        for blk in range(16):
            _, s, codes, _, _ = exact_block([float(v) for v in xs[r, blk * 16:(blk + 1) * 16]], alpha)
            assert Fr(oracle.e4m3_value(int(c.scales[r, blk]))) == s
            assert [int(v) & 7 for v in unpack(c.codes)[r, blk * 16:(blk + 1) * 16]] == [v & 7 for v in codes]


def test_amax_argument_overrides():
    x = _rand(12, (16, 64))
    am = float(np.abs(x).max()) * 2
    p = oracle.quantize(x, ROW16, FOUR_OVER_SIX, amax=am)
    assert p.alpha == oracle.global_scale(am)


def test_tile16_transpose_is_exact():
    # the packed transpose moves every element and tile scale: dequantize
    # commutes with it, and two transposes are the identity
    x = _rand(13, (64, 96))
    p = oracle.quantize(x, TILE16, FOUR_OVER_SIX)
    t = oracle.transpose_tile16(p)
    assert (t.rows, t.cols) == (96, 64)
    assert np.array_equal(oracle.dequantize(t).view(np.uint32), oracle.dequantize(p).T.copy().view(np.uint32))
    tt = oracle.transpose_tile16(t)
    assert np.array_equal(tt.codes, p.codes) and np.array_equal(tt.scales, p.scales)
    # one planted element lands at the transposed place
    y = np.zeros((32, 48), np.float32)
    y[3, 40] = 2688.0               # alpha = 1: both values are exactly representable
    y[0, 0] = -3.0
    q = oracle.transpose_tile16(oracle.quantize(y, TILE16, FOUR_OVER_SIX))
    d = oracle.dequantize(q)
    assert d[40, 3] == np.float32(2688.0) and d[0, 0] == np.float32(-3.0) and np.count_nonzero(d) == 2


def test_tile16_quantize_of_transpose_matches_transpose_on_exact_blocks():
    # a tile's scale and codes do not depend on the orientation; only the
    # fp32 order of the 6-vs-4 error sum does, and exactly representable
    # tiles have no near ties
    rng = np.random.default_rng(14)
    q = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = q[rng.integers(0, 8, (48, 64))] * rng.choice([-1, 1], (48, 64)).astype(np.float32)
    x[0, 0] = 2688.0
    a = oracle.transpose_tile16(oracle.quantize(x, TILE16, FOUR_OVER_SIX))
    b = oracle.quantize(np.ascontiguousarray(x.T), TILE16, FOUR_OVER_SIX)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales) and a.alpha == b.alpha


def _hadamard16():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


@pytest.mark.parametrize("signs", [0x0000, 0xFFFF, 0xA5C3, 0x0001])
def test_rht16_integer_inputs_match_the_matrix(signs):
    # integer inputs: every butterfly sum is exact, so the fp32 result is the
    # matrix product (1/4) H16 D x itself
    rng = np.random.default_rng(signs)
    H = _hadamard16()
    d = np.array([-1 if (signs >> i) & 1 else 1 for i in range(16)], np.int64)
    for _ in range(20):
        x = rng.integers(-1000, 1000, 16)
        want = (H @ (d * x)).astype(np.float64) / 4.0
        got = oracle.rht16(x.astype(np.float32), signs)
        assert np.array_equal(got.astype(np.float64), want)


def test_rht16_is_orthogonal_and_bounded():
    rng = np.random.default_rng(31)
    H = _hadamard16().astype(np.float64)
    signs = 0x5A0F
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    for _ in range(50):
        x = (rng.standard_normal(16) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        y = oracle.rht16(x, signs)
        exact = H @ (d * x.astype(np.float64)) / 4.0
        # four rounded stages: each adds at most 2^-24 of a partial sum <= sum |x|
        assert np.max(np.abs(y - exact)) <= 4 * 2.0 ** -24 * np.sum(np.abs(x))
        # norm preserved up to rounding; no output beyond sum |x| / 4
        assert abs(np.linalg.norm(y.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) <= \
            1e-6 * np.linalg.norm(x.astype(np.float64))
        assert np.max(np.abs(y)) <= np.sum(np.abs(x.astype(np.float64))) / 4.0 * (1 + 1e-6)
    # the inverse (D H / 4) undoes it exactly on integers
    x = rng.integers(-500, 500, 16).astype(np.float32)
    back = oracle.rht16(oracle.rht16(x, signs), 0)
    back = np.where(d < 0, -back, back)
    assert np.array_equal(back, x)


def test_col16_rht_quantizes_the_transformed_tensor():
    x = _rand(32, (64, 40))
    signs = 0x9C31
    t = np.empty_like(x)
    for c in range(x.shape[1]):
        for rb in range(x.shape[0] // 16):
            t[rb * 16:(rb + 1) * 16, c] = oracle.rht16(x[rb * 16:(rb + 1) * 16, c], signs)
    a = oracle.quantize_col16_rht(x, signs)
    b = oracle.quantize(t, COL16, FOUR_OVER_SIX)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales) and a.alpha == b.alpha


def test_rht_wgrad_product_unchanged_before_quantization():
    # (R dY)^T (R X) = dY^T X: checked on the transformed fp32 tensors in fp64
    rng = np.random.default_rng(33)
    dy = rng.standard_normal((48, 24)).astype(np.float32)
    x = rng.standard_normal((48, 20)).astype(np.float32)
    signs = 0x3E91

    def rot(m):
        out = np.empty_like(m)
        for c in range(m.shape[1]):
            for rb in range(m.shape[0] // 16):
                out[rb * 16:(rb + 1) * 16, c] = oracle.rht16(m[rb * 16:(rb + 1) * 16, c], signs)
        return out.astype(np.float64)
    got = rot(dy).T @ rot(x)
    want = dy.astype(np.float64).T @ x.astype(np.float64)
    assert np.max(np.abs(got - want)) <= 1e-5 * np.max(np.abs(want))


def test_kv_smooth_closed_forms():
    # integer keys: every partial sum is exact, so the mean is the exact mean
    # rounded once, and a constant offset added to a vector leaves the smoothed
    # vector unchanged when the mean stays exact
    rng = np.random.default_rng(40)
    k = rng.integers(-200, 200, (32, 128)).astype(np.float32)
    k[:, 0] += (128 * 7 - k.sum(axis=1))            # make every sum 896 = 7 * 128: mean exactly 7
    ks, m = oracle.kv_smooth(k)
    assert np.all(m == np.float32(7.0))
    assert np.array_equal(ks, k - np.float32(7.0))
    ks2, m2 = oracle.kv_smooth(k + np.float32(64.0))
    assert np.all(m2 == np.float32(71.0)) and np.array_equal(ks2, ks)
    # a constant vector smooths to exact zeros; a zero-mean vector is unchanged
    c = np.full((2, 64), 3.25, np.float32)
    assert not np.any(oracle.kv_smooth(c)[0])
    z = np.tile(np.array([1.0, -1.0], np.float32), (3, 32))
    zs, zm = oracle.kv_smooth(z)
    assert np.all(zm == 0) and np.array_equal(zs, z)


def test_kv_smooth_order_and_quantize():
    # random keys: the mean is within a few ulps of the fp64 mean, the
    # smoothed keys are the one-rounding differences, and the packed result is
    # the plain quantizer applied to them
    rng = np.random.default_rng(41)
    k = (rng.standard_normal((64, 128)) * 3 + rng.standard_normal((64, 1)) * 10).astype(np.float32)
    ks, m = oracle.kv_smooth(k)
    exact = k.astype(np.float64).mean(axis=1)
    assert np.all(np.abs(m - exact) <= 1e-5 * np.abs(k).sum(axis=1) / 128)
    assert np.array_equal(ks, (k - m[:, None]).astype(np.float32))
    p, m2 = oracle.kv_quantize_smoothed(k)
    q = oracle.quantize(ks, ROW16, FOUR_OVER_SIX)
    assert np.array_equal(p.codes, q.codes) and np.array_equal(p.scales, q.scales) and np.array_equal(m, m2)


def test_kv_window_pins():
    # one whole part without means is the plain dequantization; parts are
    # concatenated in order; the means are added once in fp32; bf16 output is
    # the nearest-even rounding of the fp32 window
    rng = np.random.default_rng(42)
    k1 = rng.standard_normal((40, 32)).astype(np.float32)
    k2 = rng.standard_normal((24, 32)).astype(np.float32)
    p1 = oracle.quantize(k1, ROW16, FOUR_OVER_SIX)
    p2 = oracle.quantize(k2, ROW16, FOUR_OVER_SIX)
    d1, d2 = oracle.dequantize(p1), oracle.dequantize(p2)
    assert np.array_equal(oracle.kv_window([(p1, None, 0, 40)], out_bf16=False), d1)
    w = oracle.kv_window([(p2, None, 3, 5), (p1, None, 10, 7)], out_bf16=False)
    assert np.array_equal(w, np.concatenate([d2[3:8], d1[10:17]]))
    # means that are powers of two far above the values: the add is exact
    # only in the high bits, so compare with the one-rounding fp32 sum
    means = (2.0 ** rng.integers(-3, 4, 40)).astype(np.float32)
    w = oracle.kv_window([(p1, means, 2, 30)], out_bf16=False)
    assert np.array_equal(w, (d1[2:32] + means[2:32, None]).astype(np.float32))
    # values q * 448 with a block max of 2688: alpha = 1 and s = 448 exactly,
    # so every decoded value and every sum with a small integer mean is exact
    vals = np.tile(np.array([1, 2, 3, 4, 6, 0, -1, -6], np.float32) * 448, (8, 4))
    q = oracle.quantize(vals, ROW16, FOUR_OVER_SIX)
    m8 = np.arange(8, dtype=np.float32)
    w = oracle.kv_window([(q, m8, 0, 8)], out_bf16=False)
    assert np.array_equal(w, vals + m8[:, None])
    wb = oracle.kv_window([(p2, None, 3, 5), (p1, means, 10, 7)], out_bf16=True)
    assert np.array_equal(wb, oracle.bf16_rne(oracle.kv_window([(p2, None, 3, 5), (p1, means, 10, 7)], out_bf16=False)))
