"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/nvfp4.h, and rejects bad arguments before touching the
device (validation happens before anything is enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_four_operations():
    fns = declared_functions()
    for name in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_kv_quantize"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    import nvfp4_w4a4_quantized_04_amd as m
    raw = ctypes.CDLL(m.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert sorted(m.EXPORTED) == declared_functions()
    assert m.lib.nvfp4_abi_version() == 1


def test_workspace_size_helper_names_agree():
    import nvfp4_w4a4_quantized_04_amd as m
    for rows, cols in ((16, 16), (2640, 3072), (443520, 128)):
        assert m.lib.nvfp4_workspace_size(rows, cols) == m.lib.nvfp4_quantize_workspace_size(rows, cols) > 0


def test_status_strings():
    import nvfp4_w4a4_quantized_04_amd as m
    for st in range(8):
        assert m.lib.nvfp4_status_string(st)
    assert b"scratch" in m.lib.nvfp4_status_string(7)


FAKE = 1 << 20          # an aligned non-null address that is never dereferenced


def test_quantize_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    q = m.lib.nvfp4_quantize
    # bad enums
    assert q(FAKE, 9, 16, 16, 16, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 4
    assert q(FAKE, 1, 16, 16, 16, 5, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 4
    assert q(FAKE, 1, 16, 16, 16, 0, 3, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 4
    # shapes: ROW16 needs cols % 16, TILE16 rows and cols, COL16 rows; ldx >= cols
    assert q(FAKE, 1, 16, 24, 24, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert q(FAKE, 1, 24, 16, 16, 1, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert q(FAKE, 1, 24, 16, 16, 2, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert q(FAKE, 1, 16, 32, 16, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert q(FAKE, 1, -1, 32, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    # nulls
    assert q(FAKE, 1, 16, 32, 32, 0, 1, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert q(None, 1, 16, 32, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 1
    # alignment
    assert q(FAKE + 2, 1, 16, 32, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 3
    assert q(FAKE, 1, 16, 32, 36, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 3
    # workspace needed when amax is not given
    assert q(FAKE, 1, 16, 32, 32, 0, 1, None, FAKE, FAKE, FAKE, None, 0, None) == 5
    assert q(FAKE, 1, 16, 32, 32, 0, 1, None, FAKE, FAKE, FAKE, FAKE, 16, None) == 5


def test_gemm_and_linear_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    g = m.lib.nvfp4_gemm
    ok = (FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1)
    assert g(*ok, 32, 32, 24, FAKE, 0, 32, None, None) == 2          # k % 16
    assert g(FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1, 32, 24, 32, FAKE, 0, 24, None, None) == 2  # 2D needs n % 16
    assert g(FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 1, 32, 32, 32, FAKE, 0, 32, None, None) == 4
    assert g(*ok, 32, 32, 32, FAKE, 3, 32, None, None) == 4
    assert g(*ok, 32, 32, 32, None, 0, 32, None, None) == 1
    assert g(*ok, 32, 32, 32, FAKE + 2, 0, 36, None, None) == 3       # fp32 C needs 4-byte alignment
    assert g(*ok, 32, 32, 32, FAKE, 0, 36, FAKE + 2, None) == 3        # amax output needs 4-byte alignment
    # each packed operand below 4 GiB (32-bit offsets in the GEMM's producer waves)
    assert g(*ok, 1 << 20, 32, 1 << 13, FAKE, 0, 32, None, None) == 2       # A: 2^20 rows x 2^12 bytes
    assert g(*ok, 32, 1 << 20, 1 << 13, FAKE, 0, 1 << 20, None, None) == 2  # B
    assert g(*ok, 1 << 27, 1 << 23, 16, FAKE, 0, 1 << 23, None, None) == 2  # 2^23 tiles of 128 x 128
    assert m.lib.nvfp4_linear(FAKE, 1, 1 << 20, 1 << 13, 1 << 13, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None,
                              FAKE, 1 << 40, None) == 2
    lin = m.lib.nvfp4_linear
    assert lin(FAKE, 1, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, FAKE, 10, None) == 5
    need = m.lib.nvfp4_linear_workspace_size(32, 64)
    assert need >= 32 * 64 * 9 // 16
    assert lin(FAKE, 1, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, 1, 48, None, FAKE + 16, need, None) == 3
    w = m.lib.nvfp4_wgrad
    assert w(FAKE, FAKE, 1, 24, 32, 32, 32, 32, 1, -1, None, None, FAKE, 0, 32, FAKE, 1 << 30, None) == 2   # tokens % 16
    assert w(FAKE, FAKE, 1, 32, 32, 32, 32, 32, 1, 0x10000, None, None, FAKE, 0, 32, FAKE, 1 << 30, None) == 4  # signs
    assert w(FAKE, FAKE, 1, 32, 32, 32, 32, 32, 1, -2, None, None, FAKE, 0, 32, FAKE, 1 << 30, None) == 4
    assert w(FAKE, FAKE, 1, 32, 32, 32, 32, 32, 1, -1, FAKE + 2, None, FAKE, 0, 32, FAKE, 1 << 30, None) == 3  # amax alignment
    assert w(FAKE, FAKE, 1, 1 << 23, 1 << 10, 32, 1 << 10, 32, 1, -1, None, None, FAKE, 0, 32, FAKE, 1 << 40, None) == 2
    r = m.lib.nvfp4_quantize_col16_rht
    assert r(FAKE, 1, 32, 32, 32, 1, -1, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == 4     # transform required
    assert r(FAKE, 1, 24, 32, 32, 1, 7, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == 2      # rows % 16
    assert r(FAKE, 1, 32, 32, 32, 1, 7, None, FAKE, FAKE, FAKE, None, 0, None) == 5         # workspace


def test_kv_quantize_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    assert m.lib.nvfp4_kv_quantize(FAKE, 1, 100, 120, 1, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == 2
    assert m.lib.nvfp4_kv_quantize(FAKE, 1, 100, 128, 1, None, FAKE, FAKE, FAKE, None, 0, None) == 5


def test_transpose_tile16_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    t = m.lib.nvfp4_transpose_tile16
    assert t(FAKE, FAKE, FAKE, 24, 32, FAKE, FAKE, FAKE, None) == 2        # rows % 16
    assert t(FAKE, FAKE, FAKE, 32, 40, FAKE, FAKE, FAKE, None) == 2        # cols % 16
    assert t(FAKE, FAKE, FAKE, -16, 32, FAKE, FAKE, FAKE, None) == 2
    assert t(FAKE, FAKE, None, 32, 32, FAKE, FAKE, FAKE, None) == 1        # alpha
    assert t(FAKE, None, FAKE, 32, 32, FAKE, FAKE, FAKE, None) == 1        # scales
    assert t(FAKE, FAKE, FAKE, 32, 32, FAKE + 8, FAKE, FAKE, None) == 3    # codes_t alignment


def test_dispatch_size_limit_without_gpu():
    # one lane per 16-element block and 32-bit work-item counts: at most
    # 2^32 - 2^16 blocks; each dimension alone stays below 2^31
    import nvfp4_w4a4_quantized_04_amd as m
    big_r, big_c = 1 << 22, 1 << 14                 # 2^36 elements: 2^32 blocks
    ok_r = big_r - 64                               # 2^32 - 2^16 blocks, the largest accepted
    q = m.lib.nvfp4_quantize
    assert q(FAKE, 1, big_r, big_c, big_c, 0, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert q(FAKE, 1, ok_r, big_c, big_c, 0, 1, FAKE, FAKE, FAKE, None, None, 0, None) == 1   # shape passes
    assert q(FAKE, 1, big_r, big_c, big_c, 2, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    d = m.lib.nvfp4_dequantize
    assert d(FAKE, FAKE, FAKE, big_r, big_c, 0, FAKE, 1, big_c, None) == 2
    assert d(FAKE, FAKE, FAKE, ok_r, big_c, 0, None, 1, big_c, None) == 1
    t = m.lib.nvfp4_transpose_tile16
    assert t(FAKE, FAKE, FAKE, big_r, big_c, FAKE, FAKE, FAKE, None) == 2
    assert t(FAKE, FAKE, None, ok_r, big_c, FAKE, FAKE, FAKE, None) == 1
    k = m.lib.nvfp4_kv_quantize_smoothed
    assert k(FAKE, 1, 1 << 26, 1024, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, None) == 2
    assert k(FAKE, 1, (1 << 26) - 1024, 1024, 1, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == 1


def test_hip_build_script_loads_without_the_library():
    # the build must work on a tree where libnvfp4.so does not exist yet
    import __graft_entry__ as ge
    mod = ge._hip_build_module()
    names = [os.path.basename(p) for p in mod.sources()]
    assert {"api.hip", "gemm.hip", "lora.hip", "quant.hip", "pack.hip"} <= set(names)


def test_kv_consumer_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    q = m.lib.nvfp4_kv_quantize_smoothed
    assert q(FAKE, 1, 10, 96, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, None) == 2        # head_dim not a power of two
    assert q(FAKE, 1, 10, 128, 1, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == 1       # means
    assert q(FAKE, 1, 10, 128, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 5          # workspace
    w = m.lib.nvfp4_kv_dequantize_window
    seg = (m.KvSegment * 33)()
    for i in range(33):
        seg[i] = m.KvSegment(FAKE, FAKE, FAKE, None, 0, 4)
    assert w(seg, 33, 128, FAKE, 1, 128, None) == 2                   # too many segments
    assert w(seg, 2, 120, FAKE, 1, 128, None) == 2                    # head_dim % 16
    assert w(seg, 2, 128, FAKE, 1, 100, None) == 2                    # ldo < head_dim
    assert w(seg, 2, 128, FAKE + 8, 1, 128, None) == 3                # output alignment
    bad = (m.KvSegment * 2)(m.KvSegment(FAKE, FAKE, FAKE, None, 0, 4), m.KvSegment(None, FAKE, FAKE, None, 0, 4))
    assert w(bad, 2, 128, FAKE, 1, 128, None) == 1                    # codes NULL
    neg = (m.KvSegment * 1)(m.KvSegment(FAKE, FAKE, FAKE, None, -1, 4))
    assert w(neg, 1, 128, FAKE, 1, 128, None) == 2


def test_linear_lora_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    f = m.lib.nvfp4_linear_lora
    ok = (FAKE, 32, 64, 64, 1, FAKE, FAKE, FAKE, 1, 48, FAKE, FAKE)
    assert f(*ok, 48, 1.0, FAKE, FAKE, 1, 48, None, FAKE, 1 << 30, None) == 2      # rank not a multiple of 32
    assert f(*ok, 256, 1.0, FAKE, FAKE, 1, 48, None, FAKE, 1 << 30, None) == 2     # rank above 128
    assert f(*ok, 64, 0.0, FAKE, FAKE, 1, 48, None, FAKE, 1 << 30, None) == 2      # zero scale
    assert f(*ok, 64, 1.0, None, FAKE, 1, 48, None, FAKE, 1 << 30, None) == 1      # U buffer
    assert f(*ok, 64, 1.0, FAKE + 8, FAKE, 1, 48, None, FAKE, 1 << 30, None) == 3  # U alignment
    assert f(*ok, 64, 1.0, FAKE, FAKE, 1, 48, None, FAKE, 10, None) == 5           # workspace
    assert m.lib.nvfp4_linear_lora_workspace_size(32, 64, 64) >= m.lib.nvfp4_linear_workspace_size(32, 64) + 8 * 32 * 64 * 4


def test_no_cpu_fallback():
    import torch
    import nvfp4_w4a4_quantized_04_amd as m
    with pytest.raises(ValueError):
        m.quantize(torch.zeros(16, 16))
    # every tensor the binding hands to the library must be a device tensor
    with pytest.raises(ValueError):
        m._need_gpu(None, torch.zeros(4))


def test_kv_chunked_validation_without_gpu():
    import nvfp4_w4a4_quantized_04_amd as m
    q = m.lib.nvfp4_kv_quantize_chunked
    ws = m.lib.nvfp4_kv_chunked_workspace_size(1, 24, 18480, 128, 7040)
    assert ws >= 3 * 1024 * 4
    assert m.lib.nvfp4_kv_chunked_workspace_size(2, 24, 18480, 128, 7040) >= 2 * 3 * 1024 * 4
    ok = dict(kv=FAKE, dt=1, n=2, h=24, t=100, d=128, tpc=32, rule=1, am=None, c=FAKE, s=FAKE, a=FAKE, ws=FAKE,
              wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return q(a["kv"], a["dt"], a["n"], a["h"], a["t"], a["d"], a["tpc"], a["rule"], a["am"], a["c"], a["s"],
                 a["a"], a["ws"], a["wsb"], None)
    assert call(dt=7) == 4 and call(rule=2) == 4
    assert call(d=24) == 2 and call(d=0) == 2 and call(tpc=0) == 2 and call(h=0) == 2 and call(h=1025) == 2
    assert call(n=-1) == 2
    assert call(t=1 << 20, tpc=1) == 2                        # more than 65535 chunks
    assert call(t=40000, tpc=1) == 2                          # 2 tensors x 40000 chunks: more than 65535 units
    assert call(t=0, kv=None) == 0                            # no tokens: nothing to do
    assert call(n=0, kv=None) == 0                            # no tensors: nothing to do
    assert call(kv=None) == 1 and call(a=None) == 1
    assert call(kv=FAKE + 2) == 3 and call(a=FAKE + 2) == 3
    assert call(ws=None) == 5 and call(wsb=16) == 5
    d = m.lib.nvfp4_kv_dequantize_chunked
    assert d(FAKE, FAKE, FAKE, 2, 24, 100, 128, 32, FAKE, 5, None) == 4
    assert d(FAKE, FAKE, FAKE, 2, 24, 100, 120, 32, FAKE, 1, None) == 2
    assert d(FAKE, FAKE, None, 2, 24, 100, 128, 32, FAKE, 1, None) == 1
    assert d(FAKE, FAKE, FAKE, 2, 24, 100, 128, 32, FAKE + 8, 1, None) == 3
