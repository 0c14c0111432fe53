"""GPU: strided (row-padded) inputs and outputs give the same bits as the
contiguous call, and no store lands in the padding.  The leading dimensions
are chosen to take each store path of the GEMM epilogue: bf16 tiles staged
through LDS (ld % 8 == 0), 4-element vector stores (ld % 4 == 0), and
element stores (any other ld)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_packed_equal, dev_from_host, host_bits, packed_to_device

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")

SENTINEL = -12345.0


def _padded(rows, cols, ld, dtype):
    big = torch.full((rows, ld), SENTINEL, dtype=dtype, device="cuda")
    return big, big[:, :cols]


def _pad_untouched(big, cols):
    pad = big[:, cols:]
    return bool(torch.all(pad == SENTINEL).item())


@pytest.mark.parametrize("dtype,extra", [(torch.float32, 3), (torch.float32, 4), (torch.bfloat16, 8),
                                         (torch.bfloat16, 4), (torch.bfloat16, 1)])
def test_gemm_strided_output(dtype, extra):
    m, n, k = 300, 272, 512
    print(f"[case] gemm strided out {dtype} ld=n+{extra}", flush=True)
    rng = np.random.default_rng(extra)
    A = packed_to_device(oracle.quantize(rng.standard_normal((m, k)).astype(np.float32), oracle.ROW16, 1))
    B = packed_to_device(oracle.quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32), oracle.TILE16, 1))
    ref = nv.gemm(A, B, dtype)
    big, out = _padded(m, n, n + extra, dtype)
    nv.gemm(A, B, dtype, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert _pad_untouched(big, n)


def test_linear_strided_input_and_output():
    m, k, n = 257, 320, 144
    print("[case] linear strided x and y", flush=True)
    c = workloads.config2(m=m, k=k, n=n)
    W = packed_to_device(oracle.quantize(c["w"], oracle.TILE16, 1))
    x = dev_from_host(c["x"])
    ref = nv.linear(x, W, torch.bfloat16)
    xbig = torch.zeros((m, k + 24), dtype=torch.bfloat16, device="cuda")
    xbig[:, :k] = x
    ybig, y = _padded(m, n, n + 12, torch.bfloat16)
    nv.linear(xbig[:, :k], W, torch.bfloat16, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert _pad_untouched(ybig, n)


@pytest.mark.parametrize("extra", [1, 2])
def test_wgrad_strided(extra):
    """ld = k + 1 takes the COL16 quantizer's element loads, k + 2 its paired loads."""
    t, n, k = 1040, 96, 160
    print(f"[case] wgrad strided ld=+{extra}", flush=True)
    rng = np.random.default_rng(100 + extra)
    x = dev_from_host(workloads.f32_to_bf16_bits(rng.standard_normal((t, k)).astype(np.float32)))
    dy = dev_from_host(workloads.f32_to_bf16_bits((rng.standard_normal((t, n)) * 1e-3).astype(np.float32)))
    ref = nv.wgrad(dy, x, torch.float32)
    xb = torch.zeros((t, k + extra), dtype=torch.bfloat16, device="cuda")
    db = torch.zeros((t, n + extra), dtype=torch.bfloat16, device="cuda")
    xb[:, :k] = x
    db[:, :n] = dy
    dwbig, dw = _padded(n, k, k + 5, torch.float32)
    nv.wgrad(db[:, :n], xb[:, :k], torch.float32, out=dw)
    torch.cuda.synchronize()
    assert torch.equal(dw, ref)
    assert _pad_untouched(dwbig, k)


def _offset_view(host, dtype, offset):
    """A contiguous device view of `host` that starts `offset` elements into
    its allocation: element-aligned, not 16-byte aligned."""
    d = dev_from_host(host)
    buf = torch.zeros(d.numel() + 16, dtype=dtype, device="cuda")
    v = buf[offset:offset + d.numel()].view(d.shape)
    v.copy_(d)
    return v


@pytest.mark.parametrize("dtype,offset", [(torch.bfloat16, 1), (torch.bfloat16, 3), (torch.float32, 1),
                                          (torch.float32, 2)])
def test_col16_amax_on_element_aligned_view(dtype, offset):
    """COL16 takes element-aligned inputs; its in-call amax pass then reads
    rows element by element instead of in 16-byte vectors."""
    rows, cols = 96, 200
    print(f"[case] col16 element-aligned view {dtype} offset={offset}", flush=True)
    x = np.random.default_rng(60 + offset).standard_normal((rows, cols)).astype(np.float32)
    x[37, 11] = 9.5                                # the maximum sits mid-tensor
    host = x if dtype == torch.float32 else workloads.f32_to_bf16_bits(x)
    v = _offset_view(host, dtype, offset)
    assert v.data_ptr() % 16 != 0 and v.is_contiguous()
    got = nv.quantize(v, "col16", "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(got, oracle.quantize(host, oracle.COL16, 1), "col16 offset view")


@pytest.mark.parametrize("offset", [1, 5])
def test_wgrad_element_aligned_views(offset):
    t, n, k = 1040, 96, 160
    print(f"[case] wgrad element-aligned views offset={offset}", flush=True)
    rng = np.random.default_rng(200 + offset)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((t, k)).astype(np.float32))
    dy = workloads.f32_to_bf16_bits((rng.standard_normal((t, n)) * 1e-3).astype(np.float32))
    ref = nv.wgrad(dev_from_host(dy), dev_from_host(x), torch.float32)
    got = nv.wgrad(_offset_view(dy, torch.bfloat16, offset), _offset_view(x, torch.bfloat16, offset),
                   torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("block", [oracle.ROW16, oracle.TILE16, oracle.COL16])
def test_dequantize_strided_output(block):
    rows, cols = 64, 96
    print(f"[case] dequantize strided block={block}", flush=True)
    x = np.random.default_rng(block).standard_normal((rows, cols)).astype(np.float32)
    P = packed_to_device(oracle.quantize(x, block, 1))
    ref = nv.dequantize(P, torch.float32)
    ybig, y = _padded(rows, cols, cols + 8, torch.float32)
    nv.dequantize(P, torch.float32, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert _pad_untouched(ybig, cols)


def test_linear_lora_strided():
    m, k, n, r = 130, 256, 192, 64
    print("[case] linear_lora strided x and y", flush=True)
    rng = np.random.default_rng(7)
    x = dev_from_host(workloads.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))
    W = packed_to_device(oracle.quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32), oracle.TILE16, 1))
    la = dev_from_host(workloads.f32_to_bf16_bits((rng.standard_normal((r, k)) / 16).astype(np.float32)))
    lb = dev_from_host(workloads.f32_to_bf16_bits((rng.standard_normal((n, r)) * 0.02).astype(np.float32)))
    ref, uref = nv.linear_lora(x, W, la, lb, 0.5, torch.bfloat16)
    xbig = torch.zeros((m, k + 8), dtype=torch.bfloat16, device="cuda")
    xbig[:, :k] = x
    ybig, y = _padded(m, n, n + 4, torch.bfloat16)
    _, u = nv.linear_lora(xbig[:, :k], W, la, lb, 0.5, torch.bfloat16, out=y)
    torch.cuda.synchronize()
    assert torch.equal(u, uref)
    assert torch.equal(y, ref)
    assert _pad_untouched(ybig, n)


def test_binding_rejects_wrong_outputs():
    A = nv.quantize(torch.randn(64, 128, device="cuda"), "row16")
    B = nv.quantize(torch.randn(32, 128, device="cuda"), "row16")
    with pytest.raises(ValueError):
        nv.gemm(A, B, torch.float32, out=torch.empty(64, 31, device="cuda"))
    with pytest.raises(ValueError):
        nv.gemm(A, B, torch.float32, out=torch.empty(32, 64, device="cuda").t())
    short = nv.NVFP4Tensor(A.codes[:32], A.scales, A.alpha, 64, 128, A.block)
    with pytest.raises(ValueError):
        nv.gemm(short, B, torch.float32)
