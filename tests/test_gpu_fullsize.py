"""Full-size GPU parity on the five DiT-shaped workloads, in the launch
configuration the benchmark times (one nvfp4_linear / nvfp4_kv_quantize /
nvfp4_wgrad call on the whole tensor).

Quantizer outputs (codes, scale bytes, alpha) are compared bit-exactly over the
whole tensor.  Every GEMM output is compared WHOLE against the fp64 oracle
(relative Frobenius bound 1e-5), after a quick sampled pre-check (every row
and column of the ragged last tiles plus a random sample) that fails fast with
a precise position; bf16 outputs must equal round-to-nearest-even of the same
kernel's fp32 output everywhere.
"""
import functools
import time

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import (GEMM_RTOL, assert_packed_equal, check_lora_u, check_y_on_oracle_u, dev_from_host,
                               host_bits, lora_branch_allowance, packed_to_device, rel_frobenius)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def _samples(m, n, seed, count=3000):
    """Sample positions: the last 200 rows x random columns, random rows x the
    last 300 columns, and random interior positions."""
    rng = np.random.default_rng(seed)
    ms = [np.arange(max(0, m - 200), m).repeat(4), rng.integers(0, m, count)]
    ns = [rng.integers(0, n, len(ms[0])), rng.integers(0, n, count)]
    tail_n = np.arange(max(0, n - 300), n)
    ms.append(rng.integers(0, m, len(tail_n)))
    ns.append(tail_n)
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)


def _check_gemm(y32, y16, A, B, seed):
    m, n = y32.shape
    got_all = host_bits(y32)
    ms, ns = _samples(m, n, seed)
    ref = oracle.gemm_f64_sampled(A, B, ms, ns)
    err = rel_frobenius(got_all[ms, ns], ref)
    print(f"[parity] sampled pre-check rel Frobenius {err:.3e} over {len(ms)} outputs", flush=True)
    assert err <= GEMM_RTOL, err
    t0 = time.time()
    full = oracle.gemm_f64(A, B)
    err = rel_frobenius(got_all, full)
    print(f"[parity] whole output [{m}, {n}] rel Frobenius {err:.3e} (oracle {time.time() - t0:.1f} s)", flush=True)
    assert err <= GEMM_RTOL, err
    if not np.any(full):
        assert not np.any(got_all)
    if y16 is not None:
        assert np.array_equal(host_bits(y16), oracle.bf16_rne(got_all))


@functools.lru_cache(maxsize=1)
def _config5():
    return workloads.config5()


def _linear_case(x_bits, w_bits, seed):
    m, k = x_bits.shape
    n = w_bits.shape[0]
    print(f"[case] linear m={m} k={k} n={n}", flush=True)
    W = oracle.quantize(w_bits, oracle.TILE16, oracle.FOUR_OVER_SIX)
    A = oracle.quantize(x_bits, oracle.ROW16, oracle.FOUR_OVER_SIX)
    xd = dev_from_host(x_bits)
    Wd = nv.quantize(dev_from_host(w_bits), "tile16", "4over6")
    ad = nv.quantize(xd, "row16", "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(Wd, W, "weight tile16")
    assert_packed_equal(ad, A, "activation row16")
    y32 = nv.linear(xd, Wd, torch.float32)
    y16 = nv.linear(xd, Wd, torch.bfloat16)
    torch.cuda.synchronize()
    _check_gemm(y32, y16, A, W, seed)


def test_qkv_projection_full():
    c = workloads.config2()
    _linear_case(c["x"], c["w"], 2)


def test_ffn_pair_full():
    c = workloads.config3()
    _linear_case(c["x"], c["w_up"], 3)
    _linear_case(c["a"], c["w_down"], 31)


def test_training_forward_full():
    c = _config5()
    _linear_case(c["x"], c["w"], 5)


def test_training_wgrad_full():
    c = _config5()
    t, n = c["dy"].shape
    k = c["x"].shape[1]
    print(f"[case] wgrad t={t} n={n} k={k}", flush=True)
    A = oracle.quantize(c["dy"], oracle.COL16, oracle.FOUR_OVER_SIX)
    B = oracle.quantize(c["x"], oracle.COL16, oracle.FOUR_OVER_SIX)
    dyd, xd = dev_from_host(c["dy"]), dev_from_host(c["x"])
    Ad = nv.quantize(dyd, "col16", "4over6")
    Bd = nv.quantize(xd, "col16", "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(Ad, A, "dY col16")
    assert_packed_equal(Bd, B, "X col16")
    dw32 = nv.wgrad(dyd, xd, torch.float32)
    dw16 = nv.wgrad(dyd, xd, torch.bfloat16)
    torch.cuda.synchronize()
    _check_gemm(dw32, dw16, A, B, 55)


def test_training_wgrad_rht_full():
    """WGRAD with the random Hadamard transform on both operands, full size."""
    c = _config5()
    signs = 0xC39A
    t, n = c["dy"].shape
    k = c["x"].shape[1]
    print(f"[case] wgrad rht t={t} n={n} k={k}", flush=True)
    A = oracle.quantize_col16_rht(c["dy"], signs, oracle.FOUR_OVER_SIX)
    B = oracle.quantize_col16_rht(c["x"], signs, oracle.FOUR_OVER_SIX)
    dyd, xd = dev_from_host(c["dy"]), dev_from_host(c["x"])
    Ad = nv.quantize_col16_rht(dyd, signs, "4over6")
    Bd = nv.quantize_col16_rht(xd, signs, "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(Ad, A, "R dY col16")
    assert_packed_equal(Bd, B, "R X col16")
    dw32 = nv.wgrad(dyd, xd, torch.float32, rht_signs=signs)
    dw16 = nv.wgrad(dyd, xd, torch.bfloat16, rht_signs=signs)
    torch.cuda.synchronize()
    _check_gemm(dw32, dw16, A, B, 57)


def test_training_dgrad_full():
    """DGRAD dX = dY W of the training-shaped layer: the forward's TILE16
    weight transposed in packed form, dY [32768, 3072] quantized along the
    output features."""
    c = _config5()
    t, n = c["dy"].shape
    k = c["w"].shape[1]
    print(f"[case] dgrad t={t} n={n} k={k}", flush=True)
    W = oracle.quantize(c["w"], oracle.TILE16, oracle.FOUR_OVER_SIX)
    Wt = oracle.transpose_tile16(W)
    A = oracle.quantize(c["dy"], oracle.ROW16, oracle.FOUR_OVER_SIX)
    Wd = nv.quantize(dev_from_host(c["w"]), "tile16", "4over6")
    Wtd = nv.transpose_tile16(Wd)
    dyd = dev_from_host(c["dy"])
    torch.cuda.synchronize()
    assert_packed_equal(Wtd, Wt, "W^T tile16")
    dx32 = nv.dgrad(dyd, Wtd, torch.float32)
    dx16 = nv.dgrad(dyd, Wtd, torch.bfloat16)
    torch.cuda.synchronize()
    _check_gemm(dx32, dx16, A, Wt, 56)


def test_qkv_projection_with_lora_full():
    """The QKV projection with the rank-128 BF16 LoRA branch (alpha 128): the
    whole U against the oracle's rounding of the exact sums (outside the fp32
    rounding windows), the whole y against the reference built wholly by the
    oracle and against the reference on the kernel's U."""
    c = workloads.config2()
    m, k = c["x"].shape
    n = c["w"].shape[0]
    rng = np.random.default_rng(58)
    la = workloads.f32_to_bf16_bits((rng.standard_normal((128, k)) / np.sqrt(k)).astype(np.float32))
    lb = workloads.f32_to_bf16_bits((rng.standard_normal((n, 128)) * 0.02).astype(np.float32))
    print(f"[case] linear_lora m={m} k={k} n={n} r=128", flush=True)
    W = oracle.quantize(c["w"], oracle.TILE16, oracle.FOUR_OVER_SIX)
    A = oracle.quantize(c["x"], oracle.ROW16, oracle.FOUR_OVER_SIX)
    Wd = packed_to_device(W)
    y32, u = nv.linear_lora(dev_from_host(c["x"]), Wd, dev_from_host(la), dev_from_host(lb), 1.0, torch.float32)
    y16, _ = nv.linear_lora(dev_from_host(c["x"]), Wd, dev_from_host(la), dev_from_host(lb), 1.0, torch.bfloat16)
    torch.cuda.synchronize()
    ug = host_bits(u)
    nd = check_lora_u(ug, c["x"], la)
    print(f"[parity] U elements at a rounding window and not the oracle's: {nd} of {ug.size}", flush=True)
    base = oracle.gemm_f64(A, W)
    bf = workloads.bf16_to_f32(lb).astype(np.float64)
    got = host_bits(y32)
    uo = oracle.lora_down_bf16(c["x"], la)
    ref_o = base + workloads.bf16_to_f32(uo).astype(np.float64) @ bf.T
    err_o = check_y_on_oracle_u(got, ref_o, lora_branch_allowance(ug, uo, lb, 1.0))
    ref = base + workloads.bf16_to_f32(ug).astype(np.float64) @ bf.T
    err = rel_frobenius(got, ref)
    print(f"[parity] whole output rel Frobenius {err:.3e} (kernel U), {err_o:.3e} (oracle U)", flush=True)
    assert err <= GEMM_RTOL
    assert np.array_equal(host_bits(y16), oracle.bf16_rne(got))


def test_kv_cache_full():
    c = workloads.config4()
    for name in ("k", "v"):
        kv = c[name]
        print(f"[case] kv {name} {kv.shape}", flush=True)
        flat = kv.reshape(-1, kv.shape[-1])
        ref = oracle.quantize(flat, oracle.ROW16, oracle.FOUR_OVER_SIX)
        got = nv.kv_quantize(dev_from_host(kv), "4over6")
        y = nv.dequantize(got, torch.bfloat16)
        torch.cuda.synchronize()
        assert_packed_equal(got, ref, f"kv {name}")
        assert np.array_equal(host_bits(y), oracle.bf16_rne(oracle.dequantize(ref)))


@pytest.mark.parametrize("m,n,k", [(2640, 9216, 3056), (2640, 3072, 3120), (32768, 3072, 528), (3072, 3072, 4112)])
def test_large_tiles_ragged_k(m, n, k):
    """Every large tile shape (chosen by the launcher for these sizes) with a
    K that is not a multiple of 64 and ragged M."""
    print(f"[case] gemm m={m} n={n} k={k}", flush=True)
    g = np.random.default_rng(m + n + k)
    a = workloads.f32_to_bf16_bits(g.standard_normal((m, k)).astype(np.float32))
    b = workloads.f32_to_bf16_bits((g.standard_normal((n, k)) * 0.02).astype(np.float32))
    A = oracle.quantize(a, oracle.ROW16, oracle.FOUR_OVER_SIX)
    B = oracle.quantize(b, oracle.TILE16, oracle.FOUR_OVER_SIX)
    Ad, Bd = packed_to_device(A), packed_to_device(B)
    y32 = nv.gemm(Ad, Bd, torch.float32)
    y16 = nv.gemm(Ad, Bd, torch.bfloat16)
    torch.cuda.synchronize()
    _check_gemm(y32, y16, A, B, m * 3 + k)
