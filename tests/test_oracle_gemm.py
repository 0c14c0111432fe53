"""Pins of the oracle GEMM (CPU only).

C[m, n] = alpha_A * alpha_B * sum_k (q s)_A[m, k] (q s)_B[n, k]  -- the NVFP4
GEMM of the pages ("LongLive-2.0 ..." architecture walkthrough, section
"NVFP4 Training", "The three GEMMs of backpropagation" and
"Quantization-dequantization flow": packed operands contracted, output back
in high precision).  Pinned by one-hot operands (closed form), exact-rational
sums, a library matmul on the dequantized operands, transposition symmetry
and power-of-two linearity in the global scales.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import COL16, FOUR_OVER_SIX, ROW16, TILE16
from workloads import config1


def _qs_exact(p):
    """Exact rational (q * s) matrix of a packed operand, from its bytes."""
    ca, sa, al, s2d, rows, K = p.operand()
    e2 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            b = int(ca[r, k // 2])
            code = (b >> 4) if k & 1 else (b & 15)
            sb = int(sa[r // 16, k // 16]) if s2d else int(sa[r, k // 16])
            v = e2[code & 7] * Fr(oracle.e4m3_value(sb))
            row.append(-v if code & 8 else v)
        out.append(row)
    return out


def test_one_hot_k16_closed_form():
    # A row m has its only non-zero at k = m % 16; B row n at k = n % 16.
    # Then C[m, n] = aA aB sA sB qA qB when m % 16 == n % 16, else 0.
    M = N = 32
    rng = np.random.default_rng(0)
    xa = np.zeros((M, 16), np.float32)
    xb = np.zeros((N, 16), np.float32)
    va = rng.choice([-6, -3, 1.5, 2, 4, 6], M) * 2.0 ** rng.integers(-4, 4, M)
    vb = rng.choice([-4, -1, 0.5, 3, 6], N) * 2.0 ** rng.integers(-4, 4, N)
    # plant the amax so that alpha_A = 2^-4 and alpha_B = 2^-3 exactly; then
    # every dequantized value is exactly q * s * alpha
    va[0], vb[0] = 2688.0 / 16, 2688.0 / 8
    for m in range(M):
        xa[m, m % 16] = va[m]
    for n in range(N):
        xb[n, n % 16] = vb[n]
    A = oracle.quantize(xa, ROW16, FOUR_OVER_SIX)
    B = oracle.quantize(xb, ROW16, FOUR_OVER_SIX)
    C = oracle.gemm_f64(A, B)
    assert A.alpha == 2.0 ** -4 and B.alpha == 2.0 ** -3
    ya = oracle.dequantize(A).astype(np.float64)
    yb = oracle.dequantize(B).astype(np.float64)
    for m in range(M):
        for n in range(N):
            want = 0.0
            if m % 16 == n % 16:
                # each one-hot block holds its max, so it is exactly q * s * alpha
                want = ya[m, m % 16] * yb[n, n % 16]
                assert want != 0.0
            assert C[m, n] == want


def test_config1_exact_rational():
    c = config1()
    A = oracle.quantize(c["x"], ROW16, FOUR_OVER_SIX)
    B = oracle.quantize(c["w"], TILE16, FOUR_OVER_SIX)
    C = oracle.gemm_f64(A, B)
    qa = _qs_exact(A)
    qb = _qs_exact(B)
    aa, ab = Fr(float(A.alpha)), Fr(float(B.alpha))
    for m in range(0, 64, 3):
        for n in range(0, 64, 5):
            exact = sum(x * y for x, y in zip(qa[m], qb[n])) * aa * ab
            assert abs(Fr(C[m, n]) - exact) <= abs(exact) * Fr(1, 2 ** 50) + Fr(1, 2 ** 200)


def test_matches_numpy_matmul_on_dequantized():
    rng = np.random.default_rng(1)
    xa = rng.standard_normal((48, 96)).astype(np.float32)
    xb = (rng.standard_normal((80, 96)) * 0.02).astype(np.float32)
    A = oracle.quantize(xa, ROW16, FOUR_OVER_SIX)
    B = oracle.quantize(xb, TILE16, FOUR_OVER_SIX)
    C = oracle.gemm_f64(A, B)
    # dequantize gives RN32(q s alpha); undo alpha exactly-enough in fp64 is not
    # possible, so rebuild (q s) from the exact rationals instead
    qa = np.array([[float(v) for v in r] for r in _qs_exact(A)])
    qb = np.array([[float(v) for v in r] for r in _qs_exact(B)])
    ref = (qa @ qb.T) * float(A.alpha) * float(B.alpha)
    assert np.allclose(C, ref, rtol=1e-12, atol=0)
    # and the fp32 dequantized operands give the same product to fp32 accuracy
    y = oracle.dequantize(A).astype(np.float64) @ oracle.dequantize(B).astype(np.float64).T
    assert np.linalg.norm(y - C) <= 1e-6 * np.linalg.norm(C)


def test_transpose_symmetry_and_scale_linearity():
    rng = np.random.default_rng(2)
    xa = rng.standard_normal((32, 64)).astype(np.float32)
    xb = rng.standard_normal((48, 64)).astype(np.float32)
    A = oracle.quantize(xa, ROW16, FOUR_OVER_SIX)
    B = oracle.quantize(xb, ROW16, FOUR_OVER_SIX)
    C = oracle.gemm_f64(A, B)
    assert np.array_equal(oracle.gemm_f64(B, A), C.T)
    A2 = oracle.quantize((xa * np.float32(8.0)).astype(np.float32), ROW16, FOUR_OVER_SIX)
    assert np.array_equal(oracle.gemm_f64(A2, B), C * 8.0)


def test_wgrad_with_col16_operands():
    # dW = dY^T X: both operands quantized in 16-blocks along the token axis
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 48)).astype(np.float32)
    dy = (rng.standard_normal((64, 32)) * 1e-3).astype(np.float32)
    A = oracle.quantize(dy, COL16, FOUR_OVER_SIX)        # operand [32 x 64]
    B = oracle.quantize(x, COL16, FOUR_OVER_SIX)         # operand [48 x 64]
    C = oracle.gemm_f64(A, B)
    assert C.shape == (32, 48)
    ref = oracle.dequantize(A).astype(np.float64).T @ oracle.dequantize(B).astype(np.float64)
    assert np.linalg.norm(C - ref) <= 1e-6 * np.linalg.norm(ref)


def test_sampled_matches_full():
    c = config1()
    A = oracle.quantize(c["x"], ROW16, FOUR_OVER_SIX)
    B = oracle.quantize(c["w"], TILE16, FOUR_OVER_SIX)
    C = oracle.gemm_f64(A, B)
    ms = np.array([0, 5, 63, 17], np.int64)
    ns = np.array([3, 63, 0, 17], np.int64)
    assert np.array_equal(oracle.gemm_f64_sampled(A, B, ms, ns), C[ms, ns])


def _bf16_brute(y: float) -> int:
    """Nearest bf16 (ties to even mantissa) of a double, by search over the
    bf16 magnitudes next to |y|; the sign bit is that of y."""
    sign = 0x8000 if np.signbit(y) else 0
    a = abs(float(y))
    t = int(np.array([np.float32(a)]).view(np.uint32)[0]) >> 16
    best = None
    for c in range(max(0, t - 3), min(t + 4, 0x7F81)):
        v = float(np.array([c << 16], np.uint32).view(np.float32)[0])
        key = (abs(v - a), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]


def test_bf16_rounding_of_doubles():
    rng = np.random.default_rng(50)
    y = rng.standard_normal(5000) * 10.0 ** rng.uniform(-6, 6, 5000)
    y[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -40]   # ties, near tie
    got = oracle._bf16_rne_f64(y)
    assert list(got[:4]) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]
    assert np.array_equal(got, np.array([_bf16_brute(v) for v in y], np.uint16))
    # the subnormal range and below: the smallest bf16 subnormal is 2^-133;
    # 2^-134 is the midpoint between it and zero (ties to the even zero)
    tiny = np.array([2.0 ** -134, 2.0 ** -134 * (1 + 2.0 ** -20), -2.0 ** -134, 2.0 ** -133, 3 * 2.0 ** -134,
                     2.0 ** -126, 2.0 ** -127 * 1.5, 1e-45, -1e-45, 1e-80, -1e-80, 0.0, -0.0, 2.0 ** -140])
    want = [0x0000, 0x0001, 0x8000, 0x0001, 0x0002, 0x0080, 0x0060, 0x0000, 0x8000, 0x0000, 0x8000, 0x0000,
            0x8000, 0x0000]
    assert list(oracle._bf16_rne_f64(tiny)) == want
    assert [_bf16_brute(v) for v in tiny] == want
    rng2 = np.random.default_rng(54)
    small = rng2.standard_normal(3000) * 2.0 ** rng2.uniform(-140, -120, 3000)
    assert np.array_equal(oracle._bf16_rne_f64(small), np.array([_bf16_brute(v) for v in small], np.uint16))


def test_bf16_rne_of_floats():
    # fp32 -> bf16 (the comparison rounding of every bf16 output): brute force
    # nearest-even over the two bf16 neighbours, ties included
    rng = np.random.default_rng(53)
    y = (rng.standard_normal(3000) * 10.0 ** rng.uniform(-20, 20, 3000)).astype(np.float32)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0 * 2.0 ** -100], np.float32)
    y = np.concatenate([ties, y])
    got = oracle.bf16_rne(y)
    assert list(got[:3]) == [0x3F80, 0x3F82, 0xBF80]
    assert np.array_equal(got, np.array([_bf16_brute(float(v)) for v in y], np.uint16))


def test_lora_down_integer_closed_form():
    # small integers: every dot product is exact, U is its bf16 rounding
    rng = np.random.default_rng(51)
    x = rng.integers(-8, 9, (20, 64)).astype(np.float32)
    a = rng.integers(-8, 9, (16, 64)).astype(np.float32)
    u = oracle.lora_down_bf16(x, a)
    exact = x.astype(np.int64) @ a.astype(np.int64).T
    assert np.array_equal(u, np.array([[_bf16_brute(float(v)) for v in row] for row in exact], np.uint16))


def test_linear_lora_reduces_to_the_plain_gemm_and_adds_the_branch():
    rng = np.random.default_rng(52)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    w = (rng.standard_normal((48, 64)) * 0.02).astype(np.float32)
    A = oracle.quantize(x, ROW16, FOUR_OVER_SIX)
    W = oracle.quantize(w, TILE16, FOUR_OVER_SIX)
    u = np.zeros((32, 8), np.uint16)
    b = oracle._bf16_rne_f64(rng.standard_normal((48, 8)))
    assert np.array_equal(oracle.linear_lora_f64(A, W, u, b, 1.0), oracle.gemm_f64(A, W))
    # one-hot branch: U[i, j] = 1, B[n, j] = 2 -> adds scale * 2 at (i, n) only
    u[5, 3] = 0x3F80
    b1 = np.zeros((48, 8), np.uint16)
    b1[7, 3] = 0x4000
    diff = oracle.linear_lora_f64(A, W, u, b1, 0.5) - oracle.gemm_f64(A, W)
    want = np.zeros((32, 48))
    want[5, 7] = 1.0
    assert np.array_equal(diff, want)
