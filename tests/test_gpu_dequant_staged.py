"""GPU: the dequantizers whose dense outputs are stored through LDS as
contiguous runs (ROW16 dequantize, per-chunk KV dequantize, window rebuild
into dense rows), at sizes whose last workgroup is only partly filled.
Values bit-exact against the oracle (fp32; bf16 = round-to-nearest-even of
the oracle's fp32), and nothing written past the output: the output is the
head of a larger buffer whose rest must keep its sentinel."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_packed_equal, dev_from_host, host_bits

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")

SENTINEL = -7.0
GUARD = 4096                       # sentinel elements after the output


def _guarded(n, dtype):
    return torch.full((n + GUARD,), SENTINEL, dtype=dtype, device="cuda")


def _check(buf, n, ref32, dtype):
    got = host_bits(buf[:n])
    if dtype == torch.float32:
        assert np.array_equal(got.view(np.uint32), ref32.reshape(-1).view(np.uint32)), "fp32 values"
    else:
        assert np.array_equal(got, oracle.bf16_rne(ref32).reshape(-1)), "bf16 values"
    assert np.all(buf[n:].float().cpu().numpy() == np.float32(SENTINEL)), "written past the output"


# block counts 1, 111, 2700 (10 full workgroups + 140), 513 (2 + 1), 16384 (whole workgroups only)
@pytest.mark.parametrize("shape", [(1, 16), (37, 48), (300, 144), (513, 16), (64, 4096)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_row16_dequantize_partial_last_workgroup(shape, dtype):
    rows, cols = shape
    print(f"[case] staged dequantize shape={shape} dtype={dtype}", flush=True)
    x = workloads.random_bf16(5 + rows + cols, shape, 1.0, 0.001)
    ref = oracle.quantize(x, oracle.ROW16, 1)
    got = nv.quantize(dev_from_host(x), "row16", 1)
    buf = _guarded(rows * cols, dtype)
    nv.dequantize(got, dtype, out=buf[:rows * cols].view(rows, cols))
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"quantize {shape}")
    _check(buf, rows * cols, oracle.dequantize(ref), dtype)


@pytest.mark.parametrize("dims", [(2, 3, 37, 48, 10), (1, 1, 1, 16, 1), (2, 5, 61, 128, 16)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kv_dequantize_chunked_partial_last_workgroup(dims, dtype):
    tensors, heads, tokens, d, tpc = dims
    print(f"[case] staged chunked dequantize dims={dims} dtype={dtype}", flush=True)
    kv = np.stack([workloads.random_bf16(40 + u, (heads, tokens, d), 1.0, 0.001) for u in range(tensors)])
    got = nv.kv_quantize_chunked(dev_from_host(kv), tpc, 1)
    n = kv.size
    buf = _guarded(n, dtype)
    nv.kv_dequantize_chunked(got, dtype, out=buf[:n].view(tensors, heads, tokens, d))
    torch.cuda.synchronize()
    ref = np.empty((tensors, heads, tokens, d), dtype=np.float32)
    for u in range(tensors):
        for t0 in range(0, tokens, tpc):
            t1 = min(t0 + tpc, tokens)
            p = oracle.quantize(np.ascontiguousarray(kv[u, :, t0:t1, :]).reshape(-1, d), oracle.ROW16, 1)
            ref[u, :, t0:t1, :] = oracle.dequantize(p).reshape(heads, t1 - t0, d)
    _check(buf, n, ref, dtype)


@pytest.mark.parametrize("d", [48, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_window_dense_rows_partial_workgroups(d, dtype):
    """Segments of random lengths (empty ones included) from chunks with key
    means (smoothed keys need a power-of-two head_dim) and without, written
    into dense rows: each segment's last workgroup is partly filled."""
    rng = np.random.default_rng(17 + d)
    rows = 83
    chunks, dev = [], []
    for i in range(3):
        x = workloads.random_bf16(500 + i + d, (rows, d), 1.0)
        if i == 0 and d & (d - 1) == 0:
            chunks.append(oracle.kv_quantize_smoothed(x))
            dev.append(nv.kv_quantize_smoothed(dev_from_host(x)))
        else:
            chunks.append((oracle.quantize(x, oracle.ROW16, 1), None))
            dev.append((nv.kv_quantize(dev_from_host(x), "4over6"), None))
    torch.cuda.synchronize()
    parts_ref, parts = [], []
    for j in range(12):
        i = int(rng.integers(0, 3))
        first = int(rng.integers(0, rows))
        count = 0 if j == 5 else int(rng.integers(0, rows - first + 1))
        parts_ref.append((chunks[i][0], chunks[i][1], first, count))
        parts.append((dev[i][0], dev[i][1], first, count))
    total = sum(p[3] for p in parts)
    print(f"[case] staged window d={d} dtype={dtype} rows={total}", flush=True)
    buf = _guarded(total * d, dtype)
    nv.kv_dequantize_window(parts, out=buf[:total * d].view(total, d))
    torch.cuda.synchronize()
    _check(buf, total * d, oracle.kv_window(parts_ref, out_bf16=False), dtype)
