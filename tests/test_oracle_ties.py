"""The oracle on the tie-driving tensors (CPU): at exact E2M1 midpoints, one
ulp either side, and at exact E4M3 midpoints (subnormal range included), its
codes and scale bytes are the closed-form round-to-nearest-even values that
the format's definition gives ("LongLive-2.0 ..." architecture walkthrough,
NVFP4 Training section, "NVFP4 numeric format" and "Quantization rule for a
tensor block"; ties to even and saturation are readings R5, R6)."""
import numpy as np
import pytest

import oracle
from tests.exact import E4M3, Fr, nearest_even
from tests.ties import e2m1_tie_tensor, e4m3_tie_tensor, to_input, unpack_codes


@pytest.mark.parametrize("bf16", [False, True])
def test_oracle_e2m1_midpoints_closed_form(bf16):
    x, want_codes, want_sb = e2m1_tie_tensor(bf16)
    p = oracle.quantize(to_input(x, bf16), oracle.ROW16, oracle.STATIC6)
    assert p.alpha == 1.0
    nib = unpack_codes(p.codes)
    for r in range(1, x.shape[0]):
        assert p.scales[r, 0] == want_sb[r]
        assert list(nib[r]) == list(want_codes[r]), r


def test_oracle_e4m3_midpoints_closed_form():
    x, targets = e4m3_tie_tensor(0)
    p = oracle.quantize(x, oracle.ROW16, oracle.STATIC6)
    assert p.alpha == 1.0
    n = 0
    for r, t in enumerate(targets):
        if t is None:
            continue
        assert p.scales[r, 0] == nearest_even(Fr(float(t)), E4M3), (r, t)
        n += 1
    assert n > 3 * 126 * 0.9
    # the exact midpoint 2^-10 between 0 and the smallest subnormal ties to 0:
    # a zero scale, so every code of the block is a signed zero
    r = [i for i, t in enumerate(targets) if t is not None and t == 2.0 ** -10][0]
    assert p.scales[r, 0] == 0
    assert np.all(unpack_codes(p.codes)[r] & 7 == 0)


def test_oracle_e4m3_saturating_candidate():
    # max / 4 in 448 ... 672: the 4-candidate's scale saturates at 448 (byte
    # 0x7E); for an all-equal block of 1800 it reconstructs 1792 against
    # 6 * 288 = 1728 for the 6-candidate, so it is chosen
    x = np.zeros((2, 16), np.float32)
    x[0, 0] = 2688.0
    x[1, :] = 1800.0
    p = oracle.quantize(x, oracle.ROW16, oracle.FOUR_OVER_SIX)
    assert p.scales[1, 0] == 0x7E
    assert np.all(unpack_codes(p.codes)[1] == 6)
