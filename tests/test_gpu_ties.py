"""The quantizer's rounding steps driven through exact ties on the GPU.

Format ("LongLive-2.0 ..." architecture walkthrough page, NVFP4 Training
section, "NVFP4 numeric format" and "Quantization rule for a tensor block"):
element values are the nearest E2M1 values of x / (s alpha), block scales the
nearest E4M3 values of max|x| / (alpha c); this library breaks ties to even
and saturates (readings R5, R6).

Every tensor below holds one element equal to 2688 = 448 * 6, so alpha = 1
exactly, and blocks whose maximum is 6 * 2^j, so s = 2^j and kappa = 2^-j are
exact: x * kappa then lands EXACTLY on each E2M1 midpoint, or one unit in the
last place either side of it.  A second family puts max / 6 (STATIC6) or
max / 4 (4OVER6) exactly on every E4M3 midpoint, one ulp either side, the
subnormal range from 2^-10 on, and 448 ... 672 for the saturating
4-candidate.  The GPU's codes and scale bytes must equal the closed-form
nearest-even values where the rule fixes them directly (STATIC6), and the
oracle's everywhere, for ROW16, COL16 and TILE16 blocks, fp32 and bf16 input,
with alpha computed on the device or handed in."""
import numpy as np
import pytest
import torch

import oracle
from tests.exact import E4M3, Fr, nearest_even
from tests.gpu_helpers import assert_packed_equal, dev_from_host
from tests.ties import e2m1_tie_tensor, e4m3_tie_tensor, to_input, unpack_codes

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("handed_amax", [False, True])
def test_e2m1_midpoints_row16(bf16, handed_amax):
    x, want_codes, want_sb = e2m1_tie_tensor(bf16)
    print(f"[case] e2m1 ties row16 bf16={bf16} amax_in={handed_amax} rows={x.shape[0]}", flush=True)
    xin = to_input(x, bf16)
    am = torch.tensor([2688.0], dtype=torch.float32).cuda() if handed_amax else None
    for rule in (0, 1):
        ref = oracle.quantize(xin, oracle.ROW16, rule)
        got = nv.quantize(dev_from_host(xin), "row16", rule, amax=am)
        torch.cuda.synchronize()
        assert_packed_equal(got, ref, f"e2m1 ties rule={rule}")
        if rule == 0:
            nib = unpack_codes(got.codes.cpu().numpy())
            sc = got.scales.cpu().numpy()[:, 0]
            assert got.alpha.item() == 1.0
            for r in range(1, x.shape[0]):
                assert sc[r] == want_sb[r], (r, sc[r], want_sb[r])
                assert list(nib[r]) == list(want_codes[r]), (r, list(nib[r]), list(want_codes[r]))


@pytest.mark.parametrize("bf16", [False, True])
def test_e2m1_midpoints_col16_and_tile16(bf16):
    x, want_codes, want_sb = e2m1_tie_tensor(bf16)
    # COL16: the same blocks as columns of x^T [16, rows]
    xt = np.ascontiguousarray(x.T)
    xin = to_input(xt, bf16)
    print(f"[case] e2m1 ties col16 bf16={bf16}", flush=True)
    ref = oracle.quantize(xin, oracle.COL16, 0)
    got = nv.quantize(dev_from_host(xin), "col16", 0)
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, "e2m1 ties col16")
    nib = unpack_codes(got.codes.cpu().numpy())
    for r in range(1, x.shape[0]):
        assert got.scales.cpu().numpy()[r, 0] == want_sb[r]
        assert list(nib[r]) == list(want_codes[r])
    # TILE16: 16 blocks of one j stacked into a tile (the tile max is 6 * 2^j)
    blocks = x[1:]
    groups = [blocks[i:i + 3] for i in range(0, len(blocks), 3)]          # three blocks per j
    tiles = [np.concatenate([g] * 6)[:16] for g in groups]
    xt16 = np.concatenate(tiles + [np.pad(x[:1], ((0, 15), (0, 0)))], axis=0)
    xin = to_input(np.ascontiguousarray(xt16), bf16)
    print(f"[case] e2m1 ties tile16 bf16={bf16} rows={xt16.shape[0]}", flush=True)
    for rule in (0, 1):
        ref = oracle.quantize(xin, oracle.TILE16, rule)
        got = nv.quantize(dev_from_host(xin), "tile16", rule)
        torch.cuda.synchronize()
        assert_packed_equal(got, ref, f"e2m1 ties tile16 rule={rule}")


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("block", ["row16", "col16"])
def test_e4m3_midpoints(rule, block):
    x, targets = e4m3_tie_tensor(rule)
    n_hit = sum(t is not None for t in targets)
    print(f"[case] e4m3 ties rule={rule} block={block} rows={x.shape[0]} targets={n_hit}", flush=True)
    assert n_hit > 3 * 126 * (0.9 if rule == 0 else 1.0)
    xin = np.ascontiguousarray(x.T) if block == "col16" else x
    ref = oracle.quantize(xin, oracle.BLOCKS[block], rule)
    got = nv.quantize(dev_from_host(xin), block, rule)
    torch.cuda.synchronize()
    assert_packed_equal(got, ref, f"e4m3 ties rule={rule} {block}")
    if rule == 0:
        # the scale byte is the nearest-even E4M3 value of the target itself
        sc = got.scales.cpu().numpy()[:, 0]
        for r, t in enumerate(targets):
            if t is None:
                continue
            want = nearest_even(Fr(float(t)), E4M3)
            assert sc[r] == want, (r, t, sc[r], want)
