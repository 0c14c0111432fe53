"""NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over the plain C oracle in ``nvfp4_oracle.c``.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package; the library (``nvfp4_w4a4_quantized_04_amd``) never
does, and the two share no code.

The C file states what it follows on the pages and every reading it takes.
Parity status of each function (how it is pinned, see tests/test_oracle_*.py):

  e2m1_encode / e2m1_value   pinned: exhaustive exact-rational nearest search
  e4m3_encode / e4m3_value   pinned: exhaustive exact-rational nearest search
  quantize                   pinned: exact round trips, the worked 6-vs-4
                             example, brute-force exact-rational re-derivation
                             of both candidates on small blocks, invariants
  dequantize                 pinned: exact products on representable inputs
  gemm_f64 / gemm_sampled    pinned: exact-rational sums, one-hot operands,
                             transposition symmetry
  bf16_rne                   pinned: brute-force nearest-even over the two
                             bf16 neighbours, ties included
  transpose_tile16           pinned: involution, and quantize(x^T) equals the
                             transpose on blocks whose tiles are exact
  rht16                      pinned: integer inputs against the explicit
                             (1/4) H16 D matrix product; fp32 error within
                             the four-stage bound of the fp64 product; norm
                             preserved; D H / 4 undoes it exactly on integers
  quantize_col16_rht         pinned: COL16 quantization of the tensor
                             transformed block by block with rht16
  kv_smooth                  pinned: constant vectors give zero, shift
                             invariance, mean within ulps of the fp64 mean
  kv_quantize_smoothed       pinned: ROW16 quantization of kv_smooth's output
  kv_window                  pinned: one whole part equals dequantize, parts
                             concatenated in order, exact integer sums with
                             the means, bf16 output = bf16_rne of fp32
  lora_down_bf16             pinned: integer operands (exact dot products)
                             against a brute-force bf16 rounding
  linear_lora_f64            pinned: zero branch equals gemm_f64, one-hot
                             branch adds exactly scale * U * B
  The fp32 evaluation order (readings R3/R4) is not fixed by the pages: where
  it differs from the exact-real reading (near ties) parity is unpinned and
  the rate is measured by ``quantize_exact_reading``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ROW16, TILE16, COL16 = 0, 1, 2
STATIC6, FOUR_OVER_SIX = 0, 1
BLOCKS = {"row16": ROW16, "tile16": TILE16, "col16": COL16}
RULES = {"static6": STATIC6, "4over6": FOUR_OVER_SIX}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.nvo_e2m1_encode.argtypes = [ctypes.c_float]
        L.nvo_e2m1_encode.restype = ctypes.c_int
        L.nvo_e2m1_value.argtypes = [ctypes.c_int]
        L.nvo_e2m1_value.restype = ctypes.c_double
        L.nvo_e4m3_encode.argtypes = [ctypes.c_float]
        L.nvo_e4m3_encode.restype = ctypes.c_int
        L.nvo_e4m3_value.argtypes = [ctypes.c_int]
        L.nvo_e4m3_value.restype = ctypes.c_double
        L.nvo_global_scale.argtypes = [ctypes.c_float]
        L.nvo_global_scale.restype = ctypes.c_float
        L.nvo_amax.argtypes = [P, i64, i64, i64]
        L.nvo_amax.restype = ctypes.c_float
        L.nvo_num_threads.restype = ctypes.c_int
        L.nvo_quantize.argtypes = [P, i64, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        L.nvo_quantize.restype = None
        L.nvo_quantize_exact_reading.argtypes = [P, i64, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.nvo_quantize_exact_reading.restype = None
        L.nvo_rht16.argtypes = [P, ctypes.c_uint]
        L.nvo_rht16.restype = None
        L.nvo_quantize_col16_rht.argtypes = [P, i64, i64, i64, ctypes.c_int, ctypes.c_uint, P, P, P, P, P]
        L.nvo_quantize_col16_rht.restype = None
        L.nvo_kv_smooth.argtypes = [P, i64, i64, P, P]
        L.nvo_kv_smooth.restype = None
        L.nvo_dequantize.argtypes = [P, P, ctypes.c_float, i64, i64, ctypes.c_int, P, i64]
        L.nvo_dequantize.restype = None
        L.nvo_gemm_f64.argtypes = [P, P, ctypes.c_float, ctypes.c_int, P, P, ctypes.c_float,
                                   ctypes.c_int, i64, i64, i64, P]
        L.nvo_gemm_f64.restype = ctypes.c_int
        L.nvo_gemm_f64_sampled.argtypes = [P, P, ctypes.c_float, ctypes.c_int, P, P, ctypes.c_float,
                                           ctypes.c_int, i64, P, P, i64, P]
        L.nvo_gemm_f64_sampled.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().nvo_num_threads())


# ------------------------------------------------------------- formats

def e2m1_encode(v: float) -> int:
    return int(lib().nvo_e2m1_encode(float(v)))


def e2m1_value(code: int) -> float:
    return float(lib().nvo_e2m1_value(int(code)))


def e4m3_encode(t: float) -> int:
    return int(lib().nvo_e4m3_encode(float(t)))


def e4m3_value(b: int) -> float:
    return float(lib().nvo_e4m3_value(int(b)))


def global_scale(amax: float) -> np.float32:
    return np.float32(lib().nvo_global_scale(float(amax)))


# -------------------------------------------------------------- tensors

def _as_f32(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:       # bf16 bit patterns: exact widening
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def packed_shapes(rows: int, cols: int, block: int):
    """(codes shape, scales shape) for a [rows, cols] tensor."""
    if block == ROW16:
        return (rows, cols // 2), (rows, cols // 16)
    if block == TILE16:
        return (rows, cols // 2), (rows // 16, cols // 16)
    return (cols, rows // 2), (cols, rows // 16)


class Packed:
    """codes (uint8), scales (uint8 E4M3 bytes), alpha (float32), layout."""

    def __init__(self, codes, scales, alpha, rows, cols, block, stats=None):
        self.codes, self.scales, self.alpha = codes, scales, np.float32(alpha)
        self.rows, self.cols, self.block = rows, cols, block
        self.stats = stats

    def operand(self):
        """(codes, scales, alpha, scale2d, n_rows, K) as a GEMM operand."""
        if self.block == COL16:
            return self.codes, self.scales, self.alpha, 0, self.cols, self.rows
        return self.codes, self.scales, self.alpha, int(self.block == TILE16), self.rows, self.cols


def amax(x: np.ndarray) -> np.float32:
    x = _as_f32(x)
    r, c = x.shape
    return np.float32(lib().nvo_amax(_ptr(x), r, c, c))


def quantize(x: np.ndarray, block: int = ROW16, rule: int = FOUR_OVER_SIX, amax=None) -> Packed:
    x = _as_f32(x)
    rows, cols = x.shape
    cs, ss = packed_shapes(rows, cols, block)
    codes = np.zeros(cs, np.uint8)
    scales = np.zeros(ss, np.uint8)
    alpha = np.zeros(1, np.float32)
    stats = np.zeros(2, np.int64)
    am = None if amax is None else np.array([amax], np.float32)
    lib().nvo_quantize(_ptr(x), rows, cols, cols, block, rule,
                       None if am is None else _ptr(am), _ptr(codes), _ptr(scales), _ptr(alpha), _ptr(stats))
    return Packed(codes, scales, alpha[0], rows, cols, block, stats)


def rht16(v: np.ndarray, signs: int) -> np.ndarray:
    """The 16-point random Hadamard transform of one block (fp32 steps of the
    C oracle); returns a new array."""
    out = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert out.shape == (16,)
    lib().nvo_rht16(_ptr(out), signs & 0xFFFF)
    return out


def quantize_col16_rht(x: np.ndarray, signs: int, rule: int = FOUR_OVER_SIX, amax=None) -> Packed:
    """COL16 quantization of the tensor with every 16-row column block
    transformed by rht16 (the WGRAD operand path)."""
    x = _as_f32(x)
    rows, cols = x.shape
    cs, ss = packed_shapes(rows, cols, COL16)
    codes = np.zeros(cs, np.uint8)
    scales = np.zeros(ss, np.uint8)
    alpha = np.zeros(1, np.float32)
    stats = np.zeros(2, np.int64)
    am = None if amax is None else np.array([amax], np.float32)
    lib().nvo_quantize_col16_rht(_ptr(x), rows, cols, cols, rule, signs & 0xFFFF,
                                 None if am is None else _ptr(am), _ptr(codes), _ptr(scales), _ptr(alpha),
                                 _ptr(stats))
    return Packed(codes, scales, alpha[0], rows, cols, COL16, stats)


def quantize_exact_reading(x: np.ndarray, block: int = ROW16, rule: int = FOUR_OVER_SIX) -> Packed:
    x = _as_f32(x)
    rows, cols = x.shape
    cs, ss = packed_shapes(rows, cols, block)
    codes = np.zeros(cs, np.uint8)
    scales = np.zeros(ss, np.uint8)
    alpha = np.zeros(1, np.float32)
    lib().nvo_quantize_exact_reading(_ptr(x), rows, cols, cols, block, rule, _ptr(codes), _ptr(scales), _ptr(alpha))
    return Packed(codes, scales, alpha[0], rows, cols, block)


def dequantize(p: Packed) -> np.ndarray:
    y = np.empty((p.rows, p.cols), np.float32)
    lib().nvo_dequantize(_ptr(np.ascontiguousarray(p.codes)), _ptr(np.ascontiguousarray(p.scales)),
                         float(p.alpha), p.rows, p.cols, p.block, _ptr(y), p.cols)
    return y


def gemm_f64(a: Packed, b: Packed) -> np.ndarray:
    """C[m,n] = alpha_a alpha_b sum_k Ahat[m,k] Bhat[n,k] (fp64)."""
    ca, sa, aa, a2, M, K = a.operand()
    cb, sb, ab, b2, N, Kb = b.operand()
    assert K == Kb, (K, Kb)
    C = np.empty((M, N), np.float64)
    rc = lib().nvo_gemm_f64(_ptr(np.ascontiguousarray(ca)), _ptr(np.ascontiguousarray(sa)), float(aa), a2,
                            _ptr(np.ascontiguousarray(cb)), _ptr(np.ascontiguousarray(sb)), float(ab), b2,
                            M, N, K, _ptr(C))
    if rc != 0:
        raise MemoryError("oracle gemm: allocation failed")
    return C


def gemm_f64_sampled(a: Packed, b: Packed, ms: np.ndarray, ns: np.ndarray) -> np.ndarray:
    ca, sa, aa, a2, M, K = a.operand()
    cb, sb, ab, b2, N, Kb = b.operand()
    assert K == Kb
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    assert ms.shape == ns.shape
    assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
    out = np.empty(ms.shape, np.float64)
    lib().nvo_gemm_f64_sampled(_ptr(np.ascontiguousarray(ca)), _ptr(np.ascontiguousarray(sa)), float(aa), a2,
                               _ptr(np.ascontiguousarray(cb)), _ptr(np.ascontiguousarray(sb)), float(ab), b2,
                               K, _ptr(ms), _ptr(ns), ms.size, _ptr(out))
    return out


def kv_smooth(k: np.ndarray):
    """Key smoothing of [vectors, d] keys: (smoothed keys fp32, means fp32)."""
    x = _as_f32(k)
    v, d = x.shape
    out = np.empty_like(x)
    means = np.empty(v, np.float32)
    lib().nvo_kv_smooth(_ptr(x), v, d, _ptr(out), _ptr(means))
    return out, means


def kv_quantize_smoothed(k: np.ndarray, rule: int = FOUR_OVER_SIX):
    """Smoothed keys quantized in 16-blocks along head_dim, one alpha: (Packed, means)."""
    ks, means = kv_smooth(k)
    return quantize(ks, ROW16, rule), means


def kv_window(parts, out_bf16: bool = True) -> np.ndarray:
    """The attention window the consumer reconstructs: for each part (Packed
    chunk, means or None, first vector, vector count) the dequantized rows
    [first, first + count), plus the chunk's means when given (one fp32 add),
    concatenated in order; bf16 (round to nearest even) or fp32."""
    rows = []
    for p, means, first, count in parts:
        y = dequantize(p)[first:first + count]
        if means is not None:
            y = (y + means[first:first + count, None].astype(np.float32)).astype(np.float32)
        rows.append(y)
    y = np.concatenate(rows, axis=0) if rows else np.zeros((0, 0), np.float32)
    return bf16_rne(y) if out_bf16 else y


def lora_down_bf16(x: np.ndarray, lora_a: np.ndarray) -> np.ndarray:
    """U = x A^T of the LoRA branch, rounded to bf16 (uint16 bits): x [m, k]
    and lora_a [r, k] as bf16 bits (or float32), the dot products summed in
    fp64 (every product of two bf16 values is exact) and rounded once."""
    xf = _bf16_or_f32(x).astype(np.float64)
    af = _bf16_or_f32(lora_a).astype(np.float64)
    return _bf16_rne_f64(xf @ af.T)


def linear_lora_f64(a: Packed, w: Packed, u_bf16: np.ndarray, lora_b: np.ndarray, scale: float) -> np.ndarray:
    """The W4A4 linear with a BF16 LoRA branch, in fp64: the NVFP4 product
    (gemm_f64) plus scale * U B^T, U [m, r] and lora_b [n, r] bf16 bits."""
    base = gemm_f64(a, w)
    u = _bf16_or_f32(u_bf16).astype(np.float64)
    b = _bf16_or_f32(lora_b).astype(np.float64)
    return base + float(scale) * (u @ b.T)


def _bf16_or_f32(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def bf16_rne_f64(y: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step: the
    magnitude's bf16 neighbours are compared with |y| exactly in fp64 and the
    sign is put back (subnormal bf16 values included; magnitudes below half
    the smallest subnormal give a signed zero)."""
    y = np.asarray(y, np.float64)
    sign = np.where(np.signbit(y), 0x8000, 0).astype(np.int64)
    a = np.abs(y)
    t = (a.astype(np.float32).view(np.uint32).astype(np.int64) >> 16)   # near |y|'s bf16 pattern
    cand = np.stack([t + d for d in (-2, -1, 0, 1, 2)])
    cand = np.clip(cand, 0, 0x7F80)                                     # magnitudes only: 0 ... inf
    vals = (cand.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(vals - a[None])
    best_err = err.min(axis=0)
    # among the nearest candidates take the one with an even bf16 pattern
    pick = np.where((err == best_err[None]) & ((cand & 1) == 0), cand, -1).max(axis=0)
    pick = np.where(pick < 0, np.take_along_axis(cand, err.argmin(axis=0)[None], axis=0)[0], pick)
    return (sign | pick).astype(np.uint16)


_bf16_rne_f64 = bf16_rne_f64


def transpose_tile16(p: Packed) -> Packed:
    """W^T of a TILE16-packed W, element by element: element (i, j) of W is
    element (j, i) of W^T, each 16x16 tile keeps its scale byte and the tensor
    its alpha.  Unpacks the nibbles, transposes, packs again (element 2j in
    the low nibble)."""
    if p.block != TILE16:
        raise ValueError("TILE16 tensors only")
    lo = p.codes & 0x0F
    hi = p.codes >> 4
    q = np.empty((p.rows, p.cols), np.uint8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    qt = np.ascontiguousarray(q.T)
    codes = (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)
    scales = np.ascontiguousarray(p.scales.T)
    return Packed(codes, scales, p.alpha, p.cols, p.rows, TILE16)


def bf16_rne(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, nearest-even (for comparing bf16 outputs)."""
    u = np.ascontiguousarray(y, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
