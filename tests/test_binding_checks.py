"""Host-side argument checks of the Python binding (no GPU needed): every
buffer the library writes or reads whole is checked for shape, layout and
dtype before the call, so a wrong tensor raises instead of reaching a kernel."""
import pytest
import torch

import nvfp4_w4a4_quantized_04_amd as nv


def test_check_out_shape_stride_dtype():
    nv._check_out(torch.empty(4, 8), (4, 8))
    nv._check_out(torch.empty(4, 16)[:, :8], (4, 8))                 # padded rows are fine
    nv._check_out(torch.empty(4, 8, dtype=torch.bfloat16), (4, 8))
    with pytest.raises(ValueError):
        nv._check_out(torch.empty(4, 9), (4, 8))                      # wrong shape
    with pytest.raises(ValueError):
        nv._check_out(torch.empty(8, 4).t(), (4, 8))                  # column stride 8
    with pytest.raises(ValueError):
        nv._check_out(torch.empty(32).as_strided((4, 8), (4, 1)), (4, 8))   # overlapping rows
    with pytest.raises(TypeError):
        nv._check_out(torch.empty(4, 8, dtype=torch.float16), (4, 8))
    nv._check_out(torch.empty(0, 8), (0, 8))


def test_check_packed_sizes():
    t = nv.empty_packed(32, 64, nv.ROW16, "cpu")
    nv._check_packed(t, 32, 64, nv.ROW16)
    with pytest.raises(ValueError):
        nv._check_packed(t, 32, 64, nv.TILE16)                        # wrong block
    with pytest.raises(ValueError):
        nv._check_packed(t, 16, 64, nv.ROW16)                         # wrong shape
    bad = nv.NVFP4Tensor(t.codes[:, :16], t.scales, t.alpha, 32, 64, nv.ROW16)
    with pytest.raises(ValueError):
        nv._check_packed(bad, 32, 64, nv.ROW16)                       # codes too small / not contiguous
    bad = nv.NVFP4Tensor(t.codes, t.scales.float(), t.alpha, 32, 64, nv.ROW16)
    with pytest.raises(ValueError):
        nv._check_packed(bad, 32, 64, nv.ROW16)                       # scales not uint8
    bad = nv.NVFP4Tensor(t.codes, t.scales, torch.empty(0), 32, 64, nv.ROW16)
    with pytest.raises(ValueError):
        nv._check_packed(bad, 32, 64, nv.ROW16)                       # no alpha
    c = nv.empty_packed(48, 32, nv.COL16, "cpu")                      # codes [cols][rows/2]
    assert tuple(c.codes.shape) == (32, 24) and tuple(c.scales.shape) == (32, 3)
    nv._check_packed(c, 48, 32, nv.COL16)


def test_check_vec():
    nv._check_vec(None, 1, torch.float32, "amax")
    nv._check_vec(torch.zeros(1), 1, torch.float32, "amax")
    with pytest.raises(ValueError):
        nv._check_vec(torch.zeros(1, dtype=torch.float64), 1, torch.float32, "amax")
    with pytest.raises(ValueError):
        nv._check_vec(torch.zeros(3), 4, torch.float32, "means")
