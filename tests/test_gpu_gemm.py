"""GPU parity of the NVFP4 GEMM, the fused linear (activation quantize +
GEMM) and the weight-gradient GEMM against the fp64 CPU oracle: relative
Frobenius error <= 1e-5 on fp32 outputs; bf16 outputs equal to
round-to-nearest-even of the same kernel's fp32 output."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import (GEMM_RTOL, assert_packed_equal, check_lora_u, check_y_on_oracle_u, dev_from_host,
                               host_bits, lora_branch_allowance, packed_to_device, rel_frobenius)

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def _gemm_case(a_host, b_host, a_block, b_block, seed_note=""):
    print(f"[case] gemm A{a_host.shape} B{b_host.shape} blocks={a_block},{b_block} {seed_note}", flush=True)
    A = oracle.quantize(a_host, a_block, 1)
    B = oracle.quantize(b_host, b_block, 1)
    ref = oracle.gemm_f64(A, B)
    Ad, Bd = packed_to_device(A), packed_to_device(B)
    c32 = nv.gemm(Ad, Bd, torch.float32)
    c16 = nv.gemm(Ad, Bd, torch.bfloat16)
    torch.cuda.synchronize()
    g32 = host_bits(c32)
    err = rel_frobenius(g32, ref)
    assert err <= GEMM_RTOL, err
    if not np.any(ref):
        assert not np.any(g32)
    assert np.array_equal(host_bits(c16), oracle.bf16_rne(g32))
    return err


def test_config1_tiny():
    c = workloads.config1()
    _gemm_case(c["x"], c["w"], oracle.ROW16, oracle.TILE16, "config1")


@pytest.mark.parametrize("m,n,k", [(1, 16, 16), (17, 32, 48), (64, 64, 128), (130, 96, 80), (300, 272, 1024),
                                   (513, 257, 336), (1000, 1040, 512)])
def test_shapes_1d_2d(m, n, k):
    rng = np.random.default_rng(m * 7 + n + k)
    a = workloads.f32_to_bf16_bits((rng.standard_normal((m, k))).astype(np.float32))
    b = workloads.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    nb = oracle.TILE16 if n % 16 == 0 else oracle.ROW16
    _gemm_case(a, b, oracle.ROW16, nb)


def test_both_1d_and_a_2d():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((96, 192)).astype(np.float32)
    b = rng.standard_normal((80, 192)).astype(np.float32)
    _gemm_case(a, b, oracle.ROW16, oracle.ROW16)
    _gemm_case(a, b, oracle.TILE16, oracle.TILE16)


def test_zero_operand_and_k0():
    a = np.zeros((40, 64), np.float32)
    b = np.random.default_rng(0).standard_normal((48, 64)).astype(np.float32)
    _gemm_case(a, b, oracle.ROW16, oracle.TILE16)
    Ad = nv.empty_packed(32, 0, nv.ROW16)
    Bd = nv.empty_packed(48, 0, nv.ROW16)
    Ad.alpha.fill_(1.0)
    Bd.alpha.fill_(1.0)
    c = nv.gemm(Ad, Bd, torch.float32)
    torch.cuda.synchronize()
    assert c.shape == (32, 48) and not c.any()


def test_linear_equals_quantize_then_gemm():
    c = workloads.config2(m=300, k=512, n=384)
    W = oracle.quantize(c["w"], oracle.TILE16, 1)
    Wd = packed_to_device(W)
    xd = dev_from_host(c["x"])
    y = nv.linear(xd, Wd, torch.float32)
    y16 = nv.linear(xd, Wd, torch.bfloat16)
    torch.cuda.synchronize()
    A = oracle.quantize(c["x"], oracle.ROW16, 1)
    ref = oracle.gemm_f64(A, W)
    assert rel_frobenius(host_bits(y), ref) <= GEMM_RTOL
    assert np.array_equal(host_bits(y16), oracle.bf16_rne(host_bits(y)))


def test_wgrad_col16():
    rng = np.random.default_rng(4)
    t, n, k = 1040, 96, 160
    x = workloads.f32_to_bf16_bits(rng.standard_normal((t, k)).astype(np.float32))
    dy = workloads.f32_to_bf16_bits((rng.standard_normal((t, n)) * 1e-3).astype(np.float32))
    dw = nv.wgrad(dev_from_host(dy), dev_from_host(x), torch.float32)
    torch.cuda.synchronize()
    A = oracle.quantize(dy, oracle.COL16, 1)
    B = oracle.quantize(x, oracle.COL16, 1)
    ref = oracle.gemm_f64(A, B)
    assert rel_frobenius(host_bits(dw), ref) <= GEMM_RTOL


def test_wgrad_with_handed_amax():
    """dY's and X's amax handed in (as the forward's GEMM epilogues give them)
    replace the amax passes: bit-identical dW; an amax that is not the
    tensor's max is used as given (the oracle quantized with that amax)."""
    rng = np.random.default_rng(14)
    t, n, k = 1040, 96, 160
    x0 = workloads.f32_to_bf16_bits(rng.standard_normal((t, 256)).astype(np.float32))
    w = workloads.f32_to_bf16_bits((rng.standard_normal((k, 256)) * 0.05).astype(np.float32))
    dy = workloads.f32_to_bf16_bits((rng.standard_normal((t, n)) * 1e-3).astype(np.float32))
    print("[case] wgrad handed amax", flush=True)
    # X is the output of a forward linear; its epilogue amax is max |X|
    x_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    xd = nv.linear(dev_from_host(x0), packed_to_device(oracle.quantize(w, oracle.TILE16, 1)), torch.bfloat16,
                   amax_out=x_amax)
    dyd = dev_from_host(dy)
    dy_amax = dyd.float().abs().max().reshape(1)
    ref = nv.wgrad(dyd, xd, torch.float32)
    got = nv.wgrad(dyd, xd, torch.float32, dy_amax=dy_amax, x_amax=x_amax)
    got16 = nv.wgrad(dyd, xd, torch.bfloat16, x_amax=x_amax)
    torch.cuda.synchronize()
    assert x_amax.item() == xd.float().abs().max().item()
    assert np.array_equal(host_bits(got), host_bits(ref))
    assert np.array_equal(host_bits(got16), oracle.bf16_rne(host_bits(ref)))
    # a larger amax changes alpha and the codes exactly as the oracle says
    big = x_amax * 4.0
    got_big = nv.wgrad(dyd, xd, torch.float32, x_amax=big)
    torch.cuda.synchronize()
    xh = host_bits(xd)
    A = oracle.quantize(dy, oracle.COL16, 1)
    B = oracle.quantize(xh, oracle.COL16, 1, amax=float(big.item()))
    assert rel_frobenius(host_bits(got_big), oracle.gemm_f64(A, B)) <= GEMM_RTOL
    assert not np.array_equal(host_bits(got_big), host_bits(ref))


def test_wgrad_col16_rht():
    rng = np.random.default_rng(24)
    t, n, k = 1040, 96, 160
    x = workloads.f32_to_bf16_bits(rng.standard_normal((t, k)).astype(np.float32))
    dy = workloads.f32_to_bf16_bits((rng.standard_normal((t, n)) * 1e-3).astype(np.float32))
    signs = 0x6D2B
    dw = nv.wgrad(dev_from_host(dy), dev_from_host(x), torch.float32, rht_signs=signs)
    torch.cuda.synchronize()
    A = oracle.quantize_col16_rht(dy, signs, 1)
    B = oracle.quantize_col16_rht(x, signs, 1)
    ref = oracle.gemm_f64(A, B)
    assert rel_frobenius(host_bits(dw), ref) <= GEMM_RTOL
    # the transform cancels in the product: close to the unquantized dY^T X
    exact = workloads.bf16_to_f32(dy).astype(np.float64).T @ workloads.bf16_to_f32(x).astype(np.float64)
    assert rel_frobenius(host_bits(dw), exact) < 0.2


def test_epilogue_amax_output():
    """c_amax / y_amax equal max |C| of the stored outputs (fp32 and bf16)."""
    c = workloads.config2(m=300, k=512, n=384)
    W = packed_to_device(oracle.quantize(c["w"], oracle.TILE16, 1))
    xd = dev_from_host(c["x"])
    for dt in (torch.float32, torch.bfloat16):
        am = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")   # the call must overwrite it
        y = nv.linear(xd, W, dt, amax_out=am)
        torch.cuda.synchronize()
        assert am.item() == y.float().abs().max().item()
    A = packed_to_device(oracle.quantize(c["x"], oracle.ROW16, 1))
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = nv.gemm(A, W, torch.float32, amax_out=am)
    torch.cuda.synchronize()
    assert am.item() == y.abs().max().item()


def test_kv_projection_amax_feeds_single_pass_kv_quantize():
    """K = linear(x, W_k) with the epilogue amax, then a single-pass KV
    quantize: identical to the oracle's quantization of the stored K."""
    c = workloads.config2(m=880, k=256, n=128 * 3)
    W = packed_to_device(oracle.quantize(c["w"], oracle.TILE16, 1))
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    k = nv.linear(dev_from_host(c["x"]), W, torch.bfloat16, amax_out=am)
    t1 = nv.kv_quantize(k.view(-1, 128), "4over6", amax=am)
    t2 = nv.kv_quantize(k.view(-1, 128), "4over6")
    torch.cuda.synchronize()
    ref = oracle.quantize(host_bits(k).reshape(-1, 128), oracle.ROW16, 1)
    assert_packed_equal(t1, ref, "single pass")
    assert_packed_equal(t2, ref, "two pass")


@pytest.mark.parametrize("shape", [(16, 16), (48, 160), (256, 4096), (9216, 3072), (0, 32)])
def test_transpose_tile16_bit_exact(shape):
    print(f"[case] transpose_tile16 {shape}", flush=True)
    w = workloads.random_bf16(17 + shape[0], shape, 0.02)
    W = oracle.quantize(w, oracle.TILE16, 1)
    ref = oracle.transpose_tile16(W)
    got = nv.transpose_tile16(packed_to_device(W))
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"transpose {shape}")


@pytest.mark.parametrize("m,n,k", [(300, 384, 512), (17, 64, 48), (1000, 1040, 272)])
def test_dgrad(m, n, k):
    """dX [m, k] = dY [m, n] W [n, k] through the transposed packed weight."""
    print(f"[case] dgrad m={m} n={n} k={k}", flush=True)
    rng = np.random.default_rng(m + n + k)
    dy = workloads.f32_to_bf16_bits((rng.standard_normal((m, n)) * 1e-3).astype(np.float32))
    w = workloads.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    W = oracle.quantize(w, oracle.TILE16, 1)
    Wt = nv.transpose_tile16(packed_to_device(W))
    dx = nv.dgrad(dev_from_host(dy), Wt, torch.float32)
    dx16 = nv.dgrad(dev_from_host(dy), Wt, torch.bfloat16)
    torch.cuda.synchronize()
    A = oracle.quantize(dy, oracle.ROW16, 1)
    ref = oracle.gemm_f64(A, oracle.transpose_tile16(W))
    assert rel_frobenius(host_bits(dx), ref) <= GEMM_RTOL
    assert np.array_equal(host_bits(dx16), oracle.bf16_rne(host_bits(dx)))
    # the same product on the dequantized values in the original orientation
    ref2 = oracle.dequantize(A).astype(np.float64) @ oracle.dequantize(W).astype(np.float64)
    assert rel_frobenius(host_bits(dx), ref2) <= GEMM_RTOL


@pytest.mark.parametrize("m,n,k,r", [(300, 384, 512, 128), (17, 64, 48, 32), (1000, 1040, 272, 64),
                                     (33, 257, 96, 32)])
def test_linear_lora(m, n, k, r):
    """W4A4 linear + BF16 LoRA branch: U = bf16(x A^T) equal to the oracle's
    rounding of the exact sums outside the fp32 rounding windows
    (check_lora_u); y against the reference built wholly by the oracle (its
    U), allowing only the effect of U elements inside such windows; and y
    against the reference built on the kernel's own U."""
    print(f"[case] linear_lora m={m} n={n} k={k} r={r}", flush=True)
    rng = np.random.default_rng(m + n + k + r)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    w = workloads.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    la = workloads.f32_to_bf16_bits((rng.standard_normal((r, k)) / np.sqrt(k)).astype(np.float32))
    lb = workloads.f32_to_bf16_bits((rng.standard_normal((n, r)) * 0.02).astype(np.float32))
    # N % 16 != 0 takes a 1x16-block weight (and N % 8 != 0 the unstaged bf16 epilogue)
    W = oracle.quantize(w, oracle.TILE16 if n % 16 == 0 else oracle.ROW16, 1)
    Wd = packed_to_device(W)
    scale = 0.75
    y, u = nv.linear_lora(dev_from_host(x), Wd, dev_from_host(la), dev_from_host(lb), scale, torch.float32)
    y16, _ = nv.linear_lora(dev_from_host(x), Wd, dev_from_host(la), dev_from_host(lb), scale, torch.bfloat16)
    torch.cuda.synchronize()
    ug = host_bits(u)
    nd = check_lora_u(ug, x, la)
    print(f"[parity] U elements at a rounding window and not the oracle's: {nd} of {ug.size}", flush=True)
    A = oracle.quantize(x, oracle.ROW16, 1)
    uo = oracle.lora_down_bf16(x, la)
    ref_o = oracle.linear_lora_f64(A, W, uo, lb, scale)
    check_y_on_oracle_u(host_bits(y), ref_o, lora_branch_allowance(ug, uo, lb, scale))
    ref = oracle.linear_lora_f64(A, W, ug, lb, scale)
    assert rel_frobenius(host_bits(y), ref) <= GEMM_RTOL
    assert np.array_equal(host_bits(y16), oracle.bf16_rne(host_bits(y)))


@pytest.mark.parametrize("m", [32768, 32800])
def test_linear_lora_amax_from_down_projection_limit(m):
    """The LoRA linear takes the activation amax from the down projection's
    per-workgroup maxima while there are at most 1024 of them (m = 32768,
    k = 64: 1024 row blocks of one K slice) and runs its own amax pass past
    that (m = 32800: 1025): both give the oracle's codes, hence its result."""
    k, n, r = 64, 64, 32
    print(f"[case] linear_lora amax partials m={m}", flush=True)
    rng = np.random.default_rng(m)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    x[m // 2 + 7, 5] = workloads.f32_to_bf16_bits(np.array([50.0], np.float32))[0]   # the max in a late block
    w = workloads.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    la = workloads.f32_to_bf16_bits((rng.standard_normal((r, k)) / 8).astype(np.float32))
    lb = workloads.f32_to_bf16_bits((rng.standard_normal((n, r)) * 0.02).astype(np.float32))
    W = oracle.quantize(w, oracle.TILE16, 1)
    y, u = nv.linear_lora(dev_from_host(x), packed_to_device(W), dev_from_host(la), dev_from_host(lb), 1.0,
                          torch.float32)
    torch.cuda.synchronize()
    ug = host_bits(u)
    check_lora_u(ug, x, la)
    A = oracle.quantize(x, oracle.ROW16, 1)
    uo = oracle.lora_down_bf16(x, la)
    ref_o = oracle.linear_lora_f64(A, W, uo, lb, 1.0)
    check_y_on_oracle_u(host_bits(y), ref_o, lora_branch_allowance(ug, uo, lb, 1.0))
    ref = oracle.linear_lora_f64(A, W, ug, lb, 1.0)
    assert rel_frobenius(host_bits(y), ref) <= GEMM_RTOL

