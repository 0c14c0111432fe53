"""GPU parity of the NVFP4 quantizer, dequantizer and KV quantizer against the
CPU oracle: codes, scale bytes and alpha bit-exact; dequantized fp32 values
bit-exact; bf16 output equal to round-to-nearest-even of the oracle's fp32."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_packed_equal, dev_from_host, host_bits

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")

BLOCK_NAMES = {oracle.ROW16: "row16", oracle.TILE16: "tile16", oracle.COL16: "col16"}


def _case(x_host, block, rule, amax=None):
    print(f"[case] quantize shape={x_host.shape} dtype={x_host.dtype} block={block} rule={rule}", flush=True)
    ref = oracle.quantize(x_host, block, rule, amax=amax)
    xd = dev_from_host(x_host)
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32).cuda()
    got = nv.quantize(xd, BLOCK_NAMES[block], rule, amax=am)
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"{x_host.shape} block={block} rule={rule}")
    return got, ref


@pytest.mark.parametrize("rule", [0, 1])
def test_config1_tiny(rule):
    c = workloads.config1()
    _case(c["x"], oracle.ROW16, rule)
    _case(c["w"], oracle.TILE16, rule)
    _case(c["x"], oracle.COL16, rule)


SHAPES = [(1, 16), (3, 48), (37, 160), (256, 3072), (1000, 96), (4099, 64)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("rule", [0, 1])
def test_row16_bf16_shapes(shape, rule):
    x = workloads.random_bf16(sum(shape) + rule, shape, 1.0, 0.001)
    _case(x, oracle.ROW16, rule)


@pytest.mark.parametrize("shape", [(16, 16), (48, 160), (256, 4096), (4096, 256)])
@pytest.mark.parametrize("rule", [0, 1])
def test_tile16_bf16_shapes(shape, rule):
    x = workloads.random_bf16(7 + shape[0] + rule, shape, 0.02)
    _case(x, oracle.TILE16, rule)


@pytest.mark.parametrize("shape", [(16, 1), (32, 50), (64, 257), (1024, 96), (2064, 130), (4144, 192), (160, 200),
                                   (2048, 3072)])
@pytest.mark.parametrize("rule", [0, 1])
def test_col16_bf16_shapes(shape, rule):
    x = workloads.random_bf16(11 + shape[1] + rule, shape, 1e-3, 0.001)
    _case(x, oracle.COL16, rule)


def test_col16_many_row_tiles():
    # more 128-row tiles than one grid column holds: the tile loop wraps
    x = workloads.random_bf16(12, (128 * 65535 + 48, 1), 1.0)
    _case(x, oracle.COL16, 1)


@pytest.mark.parametrize("cols", [2, 34])
def test_col16_paired_loads_across_groups(cols):
    # even column count (paired loads), 1801 groups of 16 row-blocks on 901
    # grid rows: workgroups take two groups, and the last group (5 row-blocks)
    # is a workgroup's second one, so each group's prefetch of the next is used
    rows = 16 * (16 * 1800 + 5)
    x = workloads.random_bf16(13 + cols, (rows, cols), 1.0, 0.001)
    _case(x, oracle.COL16, 1)


@pytest.mark.parametrize("shape", [(16, 1), (64, 257), (2064, 130), (4144, 192), (2048, 3072)])
@pytest.mark.parametrize("signs", [0x0000, 0xB6E3])
def test_col16_rht_bf16_shapes(shape, signs):
    print(f"[case] col16 rht shape={shape} signs={signs:#06x}", flush=True)
    x = workloads.random_bf16(19 + shape[1] + signs, shape, 1.0, 0.001)
    ref = oracle.quantize_col16_rht(x, signs, 1)
    got = nv.quantize_col16_rht(dev_from_host(x), signs, "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"col16 rht {shape} {signs:#x}")


def test_col16_rht_fp32_and_explicit_amax():
    rng = np.random.default_rng(20)
    x = (rng.standard_normal((96, 80)) * 5).astype(np.float32)
    x[7, 3] = 400.0                                  # an outlier the transform spreads over its block
    signs = 0x1F2E
    ref = oracle.quantize_col16_rht(x, signs, 1)
    got = nv.quantize_col16_rht(dev_from_host(x), signs, "4over6")
    am = float(ref.alpha) * 2688.0 * 1.5
    ref2 = oracle.quantize_col16_rht(x, signs, 1, amax=am)
    got2 = nv.quantize_col16_rht(dev_from_host(x), signs, "4over6",
                                 amax=torch.tensor([am], dtype=torch.float32).cuda())
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, "col16 rht fp32")
    assert_packed_equal(got2, ref2, "col16 rht fp32 amax")


@pytest.mark.parametrize("handed_amax", [False, True])
def test_row16_fp32_large_input_streaming_loads(handed_amax):
    # 128 MiB of fp32: at the size from which the amax and ROW16 passes read
    # with non-temporal loads (ordinary loads below it)
    rows, cols = 8192, 4096
    print(f"[case] row16 fp32 [{rows},{cols}] handed_amax={handed_amax}", flush=True)
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-3, 3, (1, cols)))).astype(np.float32)
    amax = float(np.abs(x).max()) * 1.25 if handed_amax else None
    _case(x, oracle.ROW16, 1, amax=amax)


def test_fp32_input_and_explicit_amax():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * 3).astype(np.float32)
    _case(x, oracle.ROW16, 1)
    amax = float(np.abs(x).max()) * 1.75
    _case(x, oracle.ROW16, 1, amax=amax)
    _case(x, oracle.COL16, 1, amax=amax)


def test_edge_values():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    x[0] = 0.0                      # zero block
    x[1] = -0.0                     # negative zeros
    x[2, :16] = 1e-30               # tiny next to the tensor max
    x[3] = np.float32(2.0 ** -130)  # denormals
    x[4, :16] = -np.float32(2.0 ** -140)
    x[5, 3] = 1e6                   # outlier sets amax
    x[6, :16] = np.array([6, 4.5] + [0] * 14, np.float32) * np.float32(1e6 / 2688)
    for block in (oracle.ROW16, oracle.TILE16, oracle.COL16):
        for rule in (0, 1):
            _case(x, block, rule)


@pytest.mark.parametrize("scale", [2.0 ** -90, 1e-20, 1.0, 1e20, 3e38 / 2000])
def test_extreme_magnitudes(scale):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((32, 128)) * scale).astype(np.float32)
    _case(x, oracle.ROW16, 1)
    _case(x, oracle.TILE16, 1)


def test_zero_and_empty_tensors():
    _case(np.zeros((32, 64), np.float32), oracle.ROW16, 1)
    _case(np.full((32, 64), -0.0, np.float32), oracle.COL16, 1)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    t = nv.quantize(x, "row16", "4over6")
    torch.cuda.synchronize()
    assert t.alpha.item() == 1.0 and t.codes.numel() == 0


def test_strided_rows():
    rng = np.random.default_rng(8)
    big = workloads.f32_to_bf16_bits(rng.standard_normal((40, 160)).astype(np.float32))
    xd = dev_from_host(big)[:, :96]                 # ldx = 160
    ref = oracle.quantize(np.ascontiguousarray(big[:, :96]), oracle.ROW16, 1)
    got = nv.quantize(xd, "row16", "4over6")
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, "strided")


# ------------------------------------------------------------ dequantize

@pytest.mark.parametrize("block", [oracle.ROW16, oracle.TILE16, oracle.COL16])
def test_dequantize_fp32_and_bf16(block):
    x = workloads.random_bf16(21 + block, (96, 128), 1.0, 0.001)
    got, ref = _case(x, block, 1)
    y32 = nv.dequantize(got, torch.float32)
    y16 = nv.dequantize(got, torch.bfloat16)
    torch.cuda.synchronize()
    r32 = oracle.dequantize(ref)
    assert np.array_equal(host_bits(y32).view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(host_bits(y16), oracle.bf16_rne(r32))


# ------------------------------------------------------------ KV cache

@pytest.mark.parametrize("rule", [0, 1])
def test_kv_quantize_small(rule):
    c = workloads.config4(heads=2, tokens=880)
    for name in ("k", "v"):
        kv = c[name]
        flat = kv.reshape(-1, kv.shape[-1])
        ref = oracle.quantize(flat, oracle.ROW16, rule)
        got = nv.kv_quantize(dev_from_host(kv), rule)
        torch.cuda.synchronize()
        assert_packed_equal(got, ref, f"kv {name}")
        y = nv.dequantize(got, torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), oracle.bf16_rne(oracle.dequantize(ref)))
