"""GPU parity of the KV quantizer with one global scale per chunk of tokens
(the pages' "Chunkwise quantization procedure": a per-chunk, per-layer FP32
global scale) against the oracle called once per chunk: codes, scale bytes
and every chunk's alpha bit-exact; the chunked dequantize bit-exact in fp32
and equal to the nearest-even rounding of the oracle's fp32 in bf16."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import dev_from_host, host_bits

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def _oracle_chunks(kv, tpc, rule):
    heads, tokens, d = kv.shape
    out = []
    for t0 in range(0, tokens, tpc):
        t1 = min(t0 + tpc, tokens)
        out.append((t0, t1, oracle.quantize(np.ascontiguousarray(kv[:, t0:t1, :]).reshape(-1, d), oracle.ROW16,
                                             rule)))
    return out


def _check(kv, tpc, rule, chunk_amax=False):
    heads, tokens, d = kv.shape
    print(f"[case] kv chunked heads={heads} tokens={tokens} d={d} tpc={tpc} rule={rule} dtype={kv.dtype} "
          f"amax_in={chunk_amax}", flush=True)
    refs = _oracle_chunks(kv, tpc, rule)
    kd = dev_from_host(kv)
    am = None
    if chunk_amax:
        am = torch.tensor([float(oracle.amax(np.ascontiguousarray(kv[:, t0:t1, :]).reshape(-1, d)))
                           for t0, t1, _ in refs], dtype=torch.float32).cuda()
    got = nv.kv_quantize_chunked(kd, tpc, rule, chunk_amax=am)
    y32 = nv.kv_dequantize_chunked(got, torch.float32)
    y16 = nv.kv_dequantize_chunked(got, torch.bfloat16)
    torch.cuda.synchronize()
    codes, scales = got.codes.cpu().numpy(), got.scales.cpu().numpy()
    alphas = got.alphas.cpu().numpy()
    g32, g16 = host_bits(y32), host_bits(y16)
    for c, (t0, t1, R) in enumerate(refs):
        assert alphas[c].view(np.uint32) == np.float32(R.alpha).view(np.uint32), (c, alphas[c], R.alpha)
        assert np.array_equal(scales[:, t0:t1].reshape(-1, d // 16), R.scales), f"chunk {c} scales"
        assert np.array_equal(codes[:, t0:t1].reshape(-1, d // 2), R.codes), f"chunk {c} codes"
        deq = oracle.dequantize(R)
        assert np.array_equal(g32[:, t0:t1].reshape(-1, d), deq), f"chunk {c} fp32 dequantize"
        assert np.array_equal(g16[:, t0:t1].reshape(-1, d), oracle.bf16_rne(deq)), f"chunk {c} bf16 dequantize"
    return got


@pytest.mark.parametrize("tpc", [1, 7, 16, 50, 64])
@pytest.mark.parametrize("rule", [0, 1])
def test_small_chunks(tpc, rule):
    kv = workloads.random_bf16(tpc + rule, (3, 50, 64), 1.0, 0.01)
    _check(kv.reshape(3, 50, 64), tpc, rule)


def test_fp32_input_and_magnitudes_per_chunk():
    rng = np.random.default_rng(31)
    kv = rng.standard_normal((2, 96, 32)).astype(np.float32)
    kv[:, 32:64] *= 1e-3                          # chunk 1 much smaller than chunk 0
    kv[:, 64:] *= 40.0
    got = _check(kv, 32, 1)
    a = got.alphas.cpu().numpy()
    assert a[1] < a[0] < a[2]


def test_handed_chunk_amax_and_single_chunk_equals_kv_quantize():
    kv = workloads.random_bf16(5, (4, 120, 128), 1.0, 0.001)
    _check(kv, 40, 1, chunk_amax=True)
    # one chunk covering every token: the plain KV quantizer's result
    got = nv.kv_quantize_chunked(dev_from_host(kv), 1000, "4over6")
    ref = nv.kv_quantize(dev_from_host(kv), "4over6")
    torch.cuda.synchronize()
    assert np.array_equal(got.codes.cpu().numpy().reshape(-1, 64), ref.codes.cpu().numpy())
    assert np.array_equal(got.scales.cpu().numpy().reshape(-1, 8), ref.scales.cpu().numpy())
    assert got.alphas.cpu().numpy()[0].view(np.uint32) == ref.alpha.cpu().numpy()[0].view(np.uint32)


def test_zero_chunk_and_empty():
    kv = workloads.random_bf16(6, (2, 48, 16), 1.0)
    kv[:, 16:32] = 0                              # an all-zero chunk: alpha 1, zero scales
    got = _check(kv, 16, 1)
    assert got.alphas.cpu().numpy()[1] == 1.0
    empty = torch.empty((2, 0, 16), dtype=torch.bfloat16, device="cuda")
    e = nv.kv_quantize_chunked(empty, 8)
    torch.cuda.synchronize()
    assert e.codes.numel() == 0


@pytest.mark.slow
def test_kv_cache_full_per_chunk():
    """The KV workload [24, 18480, 128] (21 latent frames of 880 tokens) with
    the pages' 8-frame chunks: chunks of 8, 8 and 5 frames, K and V."""
    c = workloads.config4()
    for name in ("k", "v"):
        _check(c[name], 8 * 880, 1)
