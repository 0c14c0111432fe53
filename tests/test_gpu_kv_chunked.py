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
    """kv [heads, tokens, d] (one tensor) or [tensors, heads, tokens, d]: every
    (tensor, chunk) unit against the oracle run on that chunk of that tensor."""
    heads, tokens, d = kv.shape[-3:]
    many = kv.ndim == 4
    print(f"[case] kv chunked shape={kv.shape} tpc={tpc} rule={rule} dtype={kv.dtype} amax_in={chunk_amax}",
          flush=True)
    per = [_oracle_chunks(t, tpc, rule) for t in (kv if many else kv[None])]
    kd = dev_from_host(kv)
    am = None
    if chunk_amax:
        am = torch.tensor([float(oracle.amax(np.ascontiguousarray(t[:, t0:t1, :]).reshape(-1, d)))
                           for t, refs in zip(kv if many else kv[None], per) for t0, t1, _ in refs],
                          dtype=torch.float32).cuda()
    got = nv.kv_quantize_chunked(kd, tpc, rule, chunk_amax=am)
    y32 = nv.kv_dequantize_chunked(got, torch.float32)
    y16 = nv.kv_dequantize_chunked(got, torch.bfloat16)
    torch.cuda.synchronize()
    codes, scales = got.codes.cpu().numpy(), got.scales.cpu().numpy()
    alphas = got.alphas.cpu().numpy()
    g32, g16 = host_bits(y32), host_bits(y16)
    if not many:
        codes, scales, alphas, g32, g16 = codes[None], scales[None], alphas[None], g32[None], g16[None]
    for u, refs in enumerate(per):
        for c, (t0, t1, R) in enumerate(refs):
            tag = f"tensor {u} chunk {c}"
            assert alphas[u, c].view(np.uint32) == np.float32(R.alpha).view(np.uint32), (tag, alphas[u, c], R.alpha)
            assert np.array_equal(scales[u, :, t0:t1].reshape(-1, d // 16), R.scales), f"{tag} scales"
            assert np.array_equal(codes[u, :, t0:t1].reshape(-1, d // 2), R.codes), f"{tag} codes"
            deq = oracle.dequantize(R)
            assert np.array_equal(g32[u, :, t0:t1].reshape(-1, d), deq), f"{tag} fp32 dequantize"
            assert np.array_equal(g16[u, :, t0:t1].reshape(-1, d), oracle.bf16_rne(deq)), f"{tag} bf16 dequantize"
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


@pytest.mark.parametrize("tpc", [5, 16, 60])
def test_two_tensors_in_one_call(tpc):
    """K and V of a layer as one [2, heads, tokens, d] input: each tensor's
    chunks get their own scales, alphas [2, n_chunks]."""
    kv = np.stack((workloads.random_bf16(40 + tpc, (3, 60, 32), 1.0, 0.01),
                   workloads.random_bf16(41 + tpc, (3, 60, 32), 50.0, 0.01)))   # V larger than K
    got = _check(kv, tpc, 1)
    a = got.alphas.cpu().numpy()
    assert a.shape == (2, (60 + tpc - 1) // tpc) and (a[1] > a[0]).all()


def test_two_tensors_handed_amax_fp32():
    rng = np.random.default_rng(33)
    kv = rng.standard_normal((2, 2, 40, 48)).astype(np.float32)
    kv[0, :, 20:] *= 1e-2
    _check(kv, 20, 0, chunk_amax=True)


@pytest.mark.slow
def test_kv_cache_full_per_chunk():
    """The KV workload [24, 18480, 128] (21 latent frames of 880 tokens) with
    the pages' 8-frame chunks: chunks of 8, 8 and 5 frames, K and V in one
    call."""
    c = workloads.config4()
    _check(np.stack((c["k"], c["v"])), 8 * 880, 1)


def test_units_at_the_limit():
    """65535 (tensor, chunk) units, the most one call takes: three tensors of
    21845 one-token chunks.  Each workgroup finds its unit's tensor and chunk
    with a multiply and shift instead of a division."""
    kv = workloads.random_bf16(77, (3, 1, 21845, 16), 1.0, 0.01)
    got = _check(kv, 1, 1)
    assert got.alphas.shape == (3, 21845)


@pytest.mark.parametrize("seed", range(8))
def test_fuzz_shapes(seed):
    """Seeded random shapes: tensors, heads, tokens, head_dim, chunk length,
    rule, input dtype and handed-in chunk maxima."""
    rng = np.random.default_rng(1000 + seed)
    tensors = int(rng.integers(1, 4))
    heads = int(rng.integers(1, 6))
    tokens = int(rng.integers(1, 301))
    d = int(rng.choice([16, 32, 48, 64, 128]))
    tpc = int(rng.integers(1, tokens + 6))
    rule = int(rng.integers(0, 2))
    shape = (tensors, heads, tokens, d)
    if rng.integers(0, 2):
        kv = workloads.random_bf16(2000 + seed, shape, float(np.exp(rng.uniform(-4, 4))), 0.01)
    else:
        kv = (rng.standard_normal(shape) * np.exp(rng.uniform(-4, 4, (1, 1, 1, d)))).astype(np.float32)
    _check(kv, tpc, rule, chunk_amax=bool(rng.integers(0, 2)))
