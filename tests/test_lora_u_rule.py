"""CPU checks of the LoRA U acceptance rule used by the GPU tests
(tests/gpu_helpers.py): a U summed in fp32 in any order and rounded once to
bf16 passes; a U with one element moved by one bf16 step where the exact sum
is far from a rounding boundary fails; so does a U whose value lies outside
the fp32 accumulation window."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import check_lora_u, lora_u_window


def _operands(seed, m=40, k=272, r=32):
    g = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(g.standard_normal((m, k)).astype(np.float32))
    la = workloads.f32_to_bf16_bits((g.standard_normal((r, k)) / np.sqrt(k)).astype(np.float32))
    return x, la


def _fp32_sum_u(x, la, order):
    """U as an fp32 accumulator would give it (products exact in fp32, sums
    rounded at each step in the given k order), rounded once to bf16."""
    xf = workloads.bf16_to_f32(x)
    af = workloads.bf16_to_f32(la)
    acc = np.zeros((x.shape[0], la.shape[0]), np.float32)
    for kk in order:
        acc = (acc + np.outer(xf[:, kk], af[:, kk]).astype(np.float32)).astype(np.float32)
    return oracle.bf16_rne(acc)


@pytest.mark.parametrize("seed", [0, 1])
def test_fp32_accumulation_in_any_order_passes(seed):
    x, la = _operands(seed)
    k = x.shape[1]
    for order in (range(k), range(k - 1, -1, -1), np.random.default_rng(seed).permutation(k)):
        check_lora_u(_fp32_sum_u(x, la, order), x, la)


def test_misrounded_element_fails():
    x, la = _operands(3)
    u = oracle.lora_down_bf16(x, la)
    lo, hi = lora_u_window(x, la)
    single = np.argwhere((lo == hi) & (u != 0))
    assert len(single) > 0.7 * u.size        # most elements are far from a boundary
    i = tuple(single[len(single) // 2])
    bad = u.copy()
    bad[i] = bad[i] + 1                      # the next bf16 value of the same sign
    with pytest.raises(AssertionError):
        check_lora_u(bad, x, la)


def test_value_outside_the_window_fails():
    x, la = _operands(4)
    u = oracle.lora_down_bf16(x, la)
    lo, hi = lora_u_window(x, la)
    pos = np.argwhere((lo != hi) & (lo < 0x8000) & (lo > 0))     # a wide window of positive values
    assert len(pos) > 0
    i = tuple(pos[0])
    bad = u.copy()
    bad[i] = hi[i] + 1                       # one bf16 step past the top of the window
    with pytest.raises(AssertionError):
        check_lora_u(bad, x, la)
    bad[i] = hi[i]                           # the top of the window itself is accepted
    check_lora_u(bad, x, la)
