"""nvfp4_linear_no_alloc: the W4A4 linear with its workspace in the library's
static per-GPU scratch, for callers that cannot allocate device memory.

GPU: two calls in a row through the C ABI -- the full QKV-projection shape,
then a smaller one (the scratch still holds the first call's contents) --
each bit-identical to nvfp4_linear on the same inputs, and within the
relative Frobenius bound of the fp64 oracle; then the largest activation
the scratch holds (32768 x 3072).  CPU: sizes beyond the scratch are refused
before anything touches the device."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import GEMM_RTOL, dev_from_host, host_bits, packed_to_device, rel_frobenius

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")

FAKE = 1 << 20          # an aligned non-null address that is never dereferenced


def test_no_alloc_refuses_sizes_beyond_the_scratch():
    f = nv.lib.nvfp4_linear_no_alloc
    assert nv.lib.nvfp4_linear_workspace_size(32768, 3072) <= nv.NO_ALLOC_SCRATCH_BYTES
    assert nv.lib.nvfp4_linear_workspace_size(32768, 4096) > nv.NO_ALLOC_SCRATCH_BYTES
    assert f(FAKE, 1, 32768, 4096, 4096, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, None) == 7
    # the argument checks of nvfp4_linear come first
    assert f(FAKE, 1, 32, 24, 24, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, None) == 2
    assert f(FAKE, 9, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, None) == 4
    assert f(None, 1, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, None) == 1
    assert f(FAKE + 2, 1, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, None) == 3


def _case(m, k, n, out_dtype, seed, check_oracle=True):
    print(f"[case] no_alloc m={m} k={k} n={n} out={out_dtype}", flush=True)
    c = workloads.config2(seed=seed, m=m, k=k, n=n)
    W = oracle.quantize(c["w"], oracle.TILE16, oracle.FOUR_OVER_SIX)
    Wd = packed_to_device(W)
    xd = dev_from_host(c["x"])
    y_ref = nv.linear(xd, Wd, out_dtype)
    am_ref = torch.zeros(1, dtype=torch.float32, device="cuda")
    nv.linear(xd, Wd, out_dtype, amax_out=am_ref)
    y = torch.full((m, n), 7.0, dtype=out_dtype, device="cuda")
    am = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    nv.linear_no_alloc(xd, Wd, y, amax_out=am)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y_ref)), "differs from nvfp4_linear"
    assert am.item() == am_ref.item()
    if check_oracle:
        A = oracle.quantize(c["x"], oracle.ROW16, oracle.FOUR_OVER_SIX)
        ref = oracle.gemm_f64(A, W)
        y32 = torch.empty((m, n), dtype=torch.float32, device="cuda")
        nv.linear_no_alloc(xd, Wd, y32)
        torch.cuda.synchronize()
        err = rel_frobenius(host_bits(y32), ref)
        print(f"[parity] no_alloc rel Frobenius {err:.3e}", flush=True)
        assert err <= GEMM_RTOL
        if out_dtype == torch.bfloat16:
            assert np.array_equal(host_bits(y), oracle.bf16_rne(host_bits(y32)))


@pytest.mark.gpu
def test_no_alloc_two_calls_match_linear():
    _case(2640, 3072, 9216, torch.bfloat16, 2)       # the QKV projection
    _case(300, 512, 384, torch.float32, 12)          # smaller, after it: stale scratch must not leak in


@pytest.mark.gpu
def test_no_alloc_largest_activation():
    _case(32768, 3072, 256, torch.bfloat16, 13, check_oracle=False)
    _case(17, 64, 48, torch.float32, 14)
