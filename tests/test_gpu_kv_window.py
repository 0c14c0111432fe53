"""GPU parity of the KV-cache consumer side against the CPU oracle: key
smoothing + quantization (codes, scales, alpha and means bit-exact), and the
one-launch window reconstruction from several cached chunks (bf16 and fp32
outputs bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_packed_equal, dev_from_host, host_bits

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def _keys(seed, vectors, d):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((vectors, d)) * 10.0 ** rng.uniform(-1, 1, (1, d)) + rng.standard_normal((vectors, 1)) * 4
    return workloads.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("vectors,d", [(1, 16), (37, 64), (880 * 2, 128), (4099, 256)])
def test_kv_quantize_smoothed(vectors, d):
    print(f"[case] kv smooth vectors={vectors} d={d}", flush=True)
    k = _keys(vectors + d, vectors, d)
    ref, ref_means = oracle.kv_quantize_smoothed(k)
    got, means = nv.kv_quantize_smoothed(dev_from_host(k))
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"smoothed {vectors}x{d}")
    assert np.array_equal(host_bits(means).view(np.uint32), ref_means.view(np.uint32))


def test_kv_quantize_smoothed_empty_and_constant():
    # no keys: only alpha is written, the oracle's 1.0 for a zero amax;
    # constant keys smooth to exact zeros
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    got, means = nv.kv_quantize_smoothed(x)
    torch.cuda.synchronize()
    ref, _ = oracle.kv_quantize_smoothed(np.zeros((0, 128), np.uint16))
    assert got.alpha.item() == ref.alpha and got.codes.numel() == 0 and means.numel() == 0
    k = workloads.f32_to_bf16_bits(np.full((33, 64), 3.5, np.float32))
    ref, ref_means = oracle.kv_quantize_smoothed(k)
    got, means = nv.kv_quantize_smoothed(dev_from_host(k))
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, "smoothed constant")
    assert np.array_equal(host_bits(means).view(np.uint32), ref_means.view(np.uint32))


def test_kv_quantize_smoothed_fp32_input():
    rng = np.random.default_rng(3)
    k = (rng.standard_normal((96, 128)) + 5).astype(np.float32)
    ref, ref_means = oracle.kv_quantize_smoothed(k)
    got, means = nv.kv_quantize_smoothed(dev_from_host(k))
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, "smoothed fp32")
    assert np.array_equal(host_bits(means).view(np.uint32), ref_means.view(np.uint32))


def test_window_from_sinks_and_recent_chunks():
    # 7 cached chunks of 2 frames x 32 tokens x 2 heads, d = 128; keys smoothed,
    # values plain; the window of the chunk starting at frame 14
    chunk_frames, frame_rows, d = 2, 32 * 2, 128
    rows = chunk_frames * frame_rows
    ks, vs, kd, vd = [], [], [], []
    for c in range(7):
        k = _keys(100 + c, rows, d)
        v = workloads.random_bf16(200 + c, (rows, d), 1.0)
        ks.append(oracle.kv_quantize_smoothed(k))
        vs.append(oracle.quantize(v, oracle.ROW16, 1))
        kd.append(nv.kv_quantize_smoothed(dev_from_host(k)))
        vd.append(nv.kv_quantize(dev_from_host(v), "4over6"))
    torch.cuda.synchronize()
    for c in range(7):
        assert_packed_equal(kd[c][0], ks[c][0], f"K chunk {c}")
        assert_packed_equal(vd[c], vs[c], f"V chunk {c}")
    runs = nv.kv_window_plan(14, chunk_frames, 6, global_sink_frames=2, shot_start=5, shot_frames=3)
    print(f"[case] window runs {runs}", flush=True)
    kparts_ref = [(ks[c][0], ks[c][1], f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    kparts = [(kd[c][0], kd[c][1], f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    vparts_ref = [(vs[c], None, f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    vparts = [(vd[c], None, f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    kw = nv.kv_dequantize_window(kparts, torch.bfloat16)
    vw = nv.kv_dequantize_window(vparts, torch.bfloat16)
    kw32 = nv.kv_dequantize_window(kparts, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kw), oracle.kv_window(kparts_ref))
    assert np.array_equal(host_bits(vw), oracle.kv_window(vparts_ref))
    assert np.array_equal(host_bits(kw32).view(np.uint32), oracle.kv_window(kparts_ref, out_bf16=False).view(np.uint32))


@pytest.mark.parametrize("d", [64, 48])
def test_window_many_segments_and_strided_output(d):
    rng = np.random.default_rng(9)
    chunks = [workloads.random_bf16(300 + i, (48, d), 1.0) for i in range(4)]
    ref = [oracle.quantize(c, oracle.ROW16, 1) for c in chunks]
    dev = [nv.kv_quantize(dev_from_host(c), "4over6") for c in chunks]
    torch.cuda.synchronize()
    parts_ref, parts = [], []
    for _ in range(nv.MAX_KV_SEGMENTS):
        i = int(rng.integers(0, 4))
        first = int(rng.integers(0, 48))
        count = int(rng.integers(0, 48 - first + 1))
        parts_ref.append((ref[i], None, first, count))
        parts.append((dev[i], None, first, count))
    total = sum(p[3] for p in parts)
    big = torch.full((total, 96), -7.0, dtype=torch.float32, device="cuda")
    out = big[:, :d]
    nv.kv_dequantize_window(parts, out=out)
    torch.cuda.synchronize()
    got = host_bits(big)
    assert np.array_equal(got[:, :d].view(np.uint32), oracle.kv_window(parts_ref, out_bf16=False).view(np.uint32))
    assert np.all(got[:, d:] == np.float32(-7.0))           # row padding untouched
