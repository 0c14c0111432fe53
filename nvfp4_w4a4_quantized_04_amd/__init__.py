"""MI355X-native NVFP4 W4A4 library -- Python binding of libnvfp4.so.

Argument marshalling only: every step of the quantizer, the dequantizer and
the GEMM runs in the HIP kernels behind the C ABI declared in
``include/nvfp4.h``.  PyTorch provides device memory and the current stream.
There is no CPU fallback: importing this module without the built library
raises, and every call requires CUDA/HIP tensors.

Names follow the pages ("LongLive-2.0: An NVFP4 Parallel Infrastructure for
Long Video Generation": ``quantize_to_fp4`` / ``fp4_dequantize`` /
``quantize_kv`` on the paper-notes page, section 3.4 and 3.6; the W4A4
linear of the architecture walkthrough page, NVFP4 Inference section).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

F32, BF16 = 0, 1
ROW16, TILE16, COL16 = 0, 1, 2
STATIC6, FOUR_OVER_SIX = 0, 1
SCALE_1D, SCALE_2D = 0, 1
_BLOCKS = {"row16": ROW16, "tile16": TILE16, "col16": COL16}
_RULES = {"static6": STATIC6, "static_6": STATIC6, "4over6": FOUR_OVER_SIX, "mse": FOUR_OVER_SIX}

STATUS = {0: "ok", 1: "null pointer", 2: "shape", 3: "alignment", 4: "dtype/enum", 5: "workspace", 6: "launch",
          7: "larger than the no-allocation scratch"}


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({STATUS.get(status, '?')})")
        self.status = status


class KvSegment(ctypes.Structure):
    """nvfp4_kv_segment_t"""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
                ("means", ctypes.c_void_p), ("first", ctypes.c_int64), ("count", ctypes.c_int64)]


MAX_KV_SEGMENTS = 32


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python nvfp4_w4a4_quantized_04_amd/build.py` "
                          "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nvfp4_abi_version.restype = i32
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_quantize_workspace_size.restype = sz
    L.nvfp4_quantize_workspace_size.argtypes = [i64, i64]
    L.nvfp4_workspace_size.restype = sz
    L.nvfp4_workspace_size.argtypes = [i64, i64]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize.argtypes = [P, i32, i64, i64, i64, i32, i32, P, P, P, P, P, sz, P]
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_dequantize.argtypes = [P, P, P, i64, i64, i32, P, i32, i64, P]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm.argtypes = [P, P, P, i32, P, P, P, i32, i64, i64, i64, P, i32, i64, P, P]
    L.nvfp4_kv_quantize.restype = i32
    L.nvfp4_kv_quantize.argtypes = [P, i32, i64, i64, i32, P, P, P, P, P, sz, P]
    L.nvfp4_linear_workspace_size.restype = sz
    L.nvfp4_linear_workspace_size.argtypes = [i64, i64]
    L.nvfp4_linear.restype = i32
    L.nvfp4_linear.argtypes = [P, i32, i64, i64, i64, i32, P, P, P, i32, i64, P, i32, i64, P, P, sz, P]
    L.nvfp4_wgrad_workspace_size.restype = sz
    L.nvfp4_wgrad_workspace_size.argtypes = [i64, i64, i64]
    L.nvfp4_wgrad.restype = i32
    L.nvfp4_wgrad.argtypes = [P, P, i32, i64, i64, i64, i64, i64, i32, i32, P, P, P, i32, i64, P, sz, P]
    L.nvfp4_kv_smooth_workspace_size.restype = sz
    L.nvfp4_kv_smooth_workspace_size.argtypes = [i64, i64]
    L.nvfp4_kv_quantize_smoothed.restype = i32
    L.nvfp4_kv_quantize_smoothed.argtypes = [P, i32, i64, i64, i32, P, P, P, P, P, sz, P]
    L.nvfp4_kv_dequantize_window.restype = i32
    L.nvfp4_kv_dequantize_window.argtypes = [ctypes.POINTER(KvSegment), i32, i64, P, i32, i64, P]
    L.nvfp4_linear_lora_workspace_size.restype = sz
    L.nvfp4_linear_lora_workspace_size.argtypes = [i64, i64, i32]
    L.nvfp4_linear_lora.restype = i32
    L.nvfp4_linear_lora.argtypes = [P, i64, i64, i64, i32, P, P, P, i32, i64, P, P, i32, ctypes.c_float, P, P, i32,
                                    i64, P, P, sz, P]
    L.nvfp4_quantize_col16_rht.restype = i32
    L.nvfp4_quantize_col16_rht.argtypes = [P, i32, i64, i64, i64, i32, i32, P, P, P, P, P, sz, P]
    L.nvfp4_transpose_tile16.restype = i32
    L.nvfp4_transpose_tile16.argtypes = [P, P, P, i64, i64, P, P, P, P]
    L.nvfp4_kv_chunked_workspace_size.restype = sz
    L.nvfp4_kv_chunked_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    L.nvfp4_kv_quantize_chunked.restype = i32
    L.nvfp4_kv_quantize_chunked.argtypes = [P, i32, i64, i64, i64, i64, i64, i32, P, P, P, P, P, sz, P]
    L.nvfp4_kv_dequantize_chunked.restype = i32
    L.nvfp4_kv_dequantize_chunked.argtypes = [P, P, P, i64, i64, i64, i64, i64, P, i32, P]
    L.nvfp4_linear_no_alloc.restype = i32
    L.nvfp4_linear_no_alloc.argtypes = [P, i32, i64, i64, i64, i32, P, P, P, i32, i64, P, i32, i64, P, P]
    return L


lib = _load()

EXPORTED = ["nvfp4_abi_version", "nvfp4_status_string", "nvfp4_quantize_workspace_size", "nvfp4_workspace_size",
            "nvfp4_quantize",
            "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_kv_quantize", "nvfp4_linear_workspace_size",
            "nvfp4_linear", "nvfp4_wgrad_workspace_size", "nvfp4_wgrad", "nvfp4_transpose_tile16",
            "nvfp4_quantize_col16_rht", "nvfp4_kv_smooth_workspace_size", "nvfp4_kv_quantize_smoothed",
            "nvfp4_kv_dequantize_window", "nvfp4_linear_lora",
            "nvfp4_linear_lora_workspace_size", "nvfp4_linear_no_alloc", "nvfp4_kv_chunked_workspace_size",
            "nvfp4_kv_quantize_chunked", "nvfp4_kv_dequantize_chunked"]

NO_ALLOC_SCRATCH_BYTES = 64 << 20      # NVFP4_NO_ALLOC_SCRATCH_BYTES


def _check(fn: str, st: int):
    if st != 0:
        raise NVFP4Error(fn, st)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _out_dtype_code(d) -> int:
    if d == torch.bfloat16:
        return BF16
    if d == torch.float32:
        return F32
    raise TypeError(f"unsupported output dtype {d}")


def _need_gpu(*ts):
    """Device tensors on the current device: the library enqueues on the
    current device's current stream and dereferences the pointers there."""
    cur = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("NVFP4 kernels need device tensors (no CPU fallback)")
        if cur is None:
            cur = torch.cuda.current_device()
        if t.device.index != cur:
            raise ValueError(f"tensor on {t.device} but the current device is cuda:{cur} "
                             "(call torch.cuda.set_device first)")


def _check_out(out: torch.Tensor, shape, what="out"):
    """A caller-supplied 2D output: exactly the shape the call writes, unit
    column stride and rows that do not overlap (a padded row stride is passed
    on to the library), float32 or bfloat16."""
    if out.dim() != 2 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(out.shape)}, the call writes {tuple(shape)}")
    if shape[0] > 0 and shape[1] > 0 and (out.stride(1) != 1 or (shape[0] > 1 and out.stride(0) < shape[1])):
        raise ValueError(f"{what} needs unit column stride and non-overlapping rows")
    _out_dtype_code(out.dtype)


def _check_vec(t, n, dtype, what):
    """A contiguous 1D buffer the library reads or writes n elements of."""
    if t is None:
        return
    if t.dtype != dtype or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of at least {n} elements")


@dataclass
class NVFP4Tensor:
    """Packed NVFP4 tensor of logical shape [rows, cols].

    codes: uint8 [rows, cols/2] (ROW16/TILE16) or [cols, rows/2] (COL16),
    element 2j in the low nibble; scales: uint8 E4M3 bytes [rows, cols/16],
    [rows/16, cols/16] or [cols, rows/16]; alpha: float32 [1]."""
    codes: torch.Tensor
    scales: torch.Tensor
    alpha: torch.Tensor
    rows: int
    cols: int
    block: int

    def operand(self):
        """(codes, scales, alpha, scale layout, operand rows, K) for nvfp4_gemm."""
        if self.block == COL16:
            return self.codes, self.scales, self.alpha, SCALE_1D, self.cols, self.rows
        return self.codes, self.scales, self.alpha, SCALE_2D if self.block == TILE16 else SCALE_1D, self.rows, self.cols


def packed_shapes(rows: int, cols: int, block: int):
    if block == ROW16:
        return (rows, cols // 2), (rows, cols // 16)
    if block == TILE16:
        return (rows, cols // 2), (rows // 16, cols // 16)
    return (cols, rows // 2), (cols, rows // 16)


def _check_packed(t: NVFP4Tensor, rows: int, cols: int, block: int, what="packed tensor"):
    """A packed tensor whose buffers the library reads or writes whole: uint8
    codes and scales of exactly the layout's sizes, contiguous, and a float32
    alpha."""
    if t.block != block or t.rows != rows or t.cols != cols:
        raise ValueError(f"{what}: block {t.block} [{t.rows}, {t.cols}], expected block {block} [{rows}, {cols}]")
    cs, ss = packed_shapes(rows, cols, block)
    for buf, shape, name in ((t.codes, cs, "codes"), (t.scales, ss, "scales")):
        if buf.dtype != torch.uint8 or not buf.is_contiguous() or buf.numel() != shape[0] * shape[1]:
            raise ValueError(f"{what}: {name} must be contiguous uint8 with {shape[0] * shape[1]} bytes")
    _check_vec(t.alpha, 1, torch.float32, f"{what}: alpha")


def empty_packed(rows: int, cols: int, block: int, device="cuda") -> NVFP4Tensor:
    cs, ss = packed_shapes(rows, cols, block)
    return NVFP4Tensor(torch.empty(cs, dtype=torch.uint8, device=device),
                       torch.empty(ss, dtype=torch.uint8, device=device),
                       torch.empty(1, dtype=torch.float32, device=device), rows, cols, block)


def _block(block) -> int:
    return _BLOCKS[block] if isinstance(block, str) else int(block)


def _rule(rule) -> int:
    return _RULES[rule] if isinstance(rule, str) else int(rule)


def quantize(x: torch.Tensor, block="row16", rule="4over6", amax: torch.Tensor | None = None,
             out: NVFP4Tensor | None = None, workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """NVFP4-quantize a 2D float32/bfloat16 device tensor (``quantize_to_fp4``)."""
    _need_gpu(x, amax)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2D with unit column stride")
    b = _block(block)
    rows, cols = x.shape
    _check_vec(amax, 1, torch.float32, "amax")
    if out is None:
        out = empty_packed(rows, cols, b, x.device)
    _check_packed(out, rows, cols, b, "out")
    if workspace is None and amax is None:
        workspace = torch.empty(lib.nvfp4_quantize_workspace_size(rows, cols), dtype=torch.uint8, device=x.device)
    wsz = 0 if workspace is None else workspace.numel()
    _need_gpu(out.codes, out.scales, out.alpha, workspace)
    _check("nvfp4_quantize", lib.nvfp4_quantize(
        _ptr(x), _dtype_code(x), rows, cols, x.stride(0), b, _rule(rule), _ptr(amax),
        _ptr(out.codes), _ptr(out.scales), _ptr(out.alpha), _ptr(workspace), wsz, _stream()))
    return out


def dequantize(t: NVFP4Tensor, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """Xhat = (q * s) * alpha in the tensor's original orientation (``fp4_dequantize``)."""
    _need_gpu(t.codes)
    _check_packed(t, t.rows, t.cols, t.block, "t")
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=dtype, device=t.codes.device)
    _check_out(out, (t.rows, t.cols))
    _need_gpu(t.scales, t.alpha, out)
    _check("nvfp4_dequantize", lib.nvfp4_dequantize(
        _ptr(t.codes), _ptr(t.scales), _ptr(t.alpha), t.rows, t.cols, t.block,
        _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _stream()))
    return out


def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
         amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """C = alpha_A alpha_B Ahat Bhat^T on packed operands.  amax_out (float32
    [1], optional) receives max |C| of the stored values."""
    ca, sa, aa, la, m, k = a.operand()
    cb, sb, ab, lb, n, kb = b.operand()
    if k != kb:
        raise ValueError(f"contraction mismatch {k} vs {kb}")
    _need_gpu(ca, cb)
    _check_packed(a, a.rows, a.cols, a.block, "a")
    _check_packed(b, b.rows, b.cols, b.block, "b")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=ca.device)
    _check_out(out, (m, n))
    _check_vec(amax_out, 1, torch.float32, "amax_out")
    _need_gpu(sa, aa, sb, ab, out, amax_out)
    _check("nvfp4_gemm", lib.nvfp4_gemm(
        _ptr(ca), _ptr(sa), _ptr(aa), la, _ptr(cb), _ptr(sb), _ptr(ab), lb, m, n, k,
        _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _ptr(amax_out), _stream()))
    return out


def kv_quantize(kv: torch.Tensor, rule="4over6", out: NVFP4Tensor | None = None,
                workspace: torch.Tensor | None = None, amax: torch.Tensor | None = None) -> NVFP4Tensor:
    """Quantize a K or V cache tensor [..., head_dim] (``quantize_kv``).  amax:
    optional device float32 [1] holding max |kv| (single pass)."""
    _need_gpu(kv)
    if not kv.is_contiguous():
        raise ValueError("kv must be contiguous")
    d = kv.shape[-1]
    vectors = kv.numel() // d if d else 0
    _check_vec(amax, 1, torch.float32, "amax")
    if out is None:
        out = empty_packed(vectors, d, ROW16, kv.device)
    _check_packed(out, vectors, d, ROW16, "out")
    if workspace is None:
        workspace = torch.empty(lib.nvfp4_quantize_workspace_size(vectors, d), dtype=torch.uint8, device=kv.device)
    _need_gpu(amax, out.codes, out.scales, out.alpha, workspace)
    _check("nvfp4_kv_quantize", lib.nvfp4_kv_quantize(
        _ptr(kv), _dtype_code(kv), vectors, d, _rule(rule), _ptr(amax), _ptr(out.codes), _ptr(out.scales),
        _ptr(out.alpha), _ptr(workspace), workspace.numel(), _stream()))
    return out


def linear_workspace(m: int, k: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib.nvfp4_linear_workspace_size(m, k), dtype=torch.uint8, device=device)


def linear(x: torch.Tensor, w: NVFP4Tensor, out_dtype=torch.bfloat16, rule="4over6",
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 forward: y = quantize(x) @ w^T with the activation quantizer fused in
    the call.  amax_out (float32 [1], optional) receives max |y|."""
    _need_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2D with unit column stride")
    cw, sw, aw, lw, n, kw = w.operand()
    m, k = x.shape
    if k != kw:
        raise ValueError(f"in_features mismatch {k} vs {kw}")
    _check_packed(w, w.rows, w.cols, w.block, "w")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check_out(out, (m, n))
    _check_vec(amax_out, 1, torch.float32, "amax_out")
    if workspace is None:
        workspace = linear_workspace(m, k, x.device)
    _need_gpu(cw, sw, aw, out, amax_out, workspace)
    _check("nvfp4_linear", lib.nvfp4_linear(
        _ptr(x), _dtype_code(x), m, k, x.stride(0), _rule(rule), _ptr(cw), _ptr(sw), _ptr(aw), lw, n,
        _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _ptr(amax_out), _ptr(workspace), workspace.numel(),
        _stream()))
    return out


def linear_no_alloc(x: torch.Tensor, w: NVFP4Tensor, out: torch.Tensor, rule="4over6",
                    amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_linear_no_alloc: the same W4A4 forward as `linear`, with the
    workspace taken from the library's static per-GPU scratch (no device
    allocation in the call; calls on one GPU must not overlap).  `out` is
    required, so the call allocates nothing on this side either."""
    _need_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2D with unit column stride")
    cw, sw, aw, lw, n, kw = w.operand()
    m, k = x.shape
    if k != kw:
        raise ValueError(f"in_features mismatch {k} vs {kw}")
    _check_packed(w, w.rows, w.cols, w.block, "w")
    _check_out(out, (m, n))
    _check_vec(amax_out, 1, torch.float32, "amax_out")
    _need_gpu(cw, sw, aw, out, amax_out)
    _check("nvfp4_linear_no_alloc", lib.nvfp4_linear_no_alloc(
        _ptr(x), _dtype_code(x), m, k, x.stride(0), _rule(rule), _ptr(cw), _ptr(sw), _ptr(aw), lw, n,
        _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _ptr(amax_out), _stream()))
    return out


def wgrad_workspace(tokens: int, n_out: int, k_in: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib.nvfp4_wgrad_workspace_size(tokens, n_out, k_in), dtype=torch.uint8, device=device)


def wgrad(dy: torch.Tensor, x: torch.Tensor, out_dtype=torch.float32, rule="4over6",
          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          rht_signs: int | None = None, dy_amax: torch.Tensor | None = None,
          x_amax: torch.Tensor | None = None) -> torch.Tensor:
    """dW = dY^T X with both operands NVFP4-quantized along the token axis;
    rht_signs (0..0xFFFF) first applies the random Hadamard transform to both.
    dy_amax / x_amax (float32 [1] device tensors, optional): the operands' max
    |.| (e.g. the forward's), replacing their amax passes."""
    _need_gpu(dy, x)
    t, n = dy.shape
    t2, k = x.shape
    if t != t2 or dy.dtype != x.dtype:
        raise ValueError("dy and x need the same token count and dtype")
    if dy.dim() != 2 or x.dim() != 2 or dy.stride(1) != 1 or x.stride(1) != 1:
        raise ValueError("dy and x must be 2D with unit column stride")
    if out is None:
        out = torch.empty((n, k), dtype=out_dtype, device=x.device)
    _check_out(out, (n, k))
    _check_vec(dy_amax, 1, torch.float32, "dy_amax")
    _check_vec(x_amax, 1, torch.float32, "x_amax")
    if workspace is None:
        workspace = wgrad_workspace(t, n, k, x.device)
    _need_gpu(out, workspace, dy_amax, x_amax)
    _check("nvfp4_wgrad", lib.nvfp4_wgrad(
        _ptr(dy), _ptr(x), _dtype_code(x), t, n, k, dy.stride(0), x.stride(0), _rule(rule),
        -1 if rht_signs is None else int(rht_signs), _ptr(dy_amax), _ptr(x_amax), _ptr(out),
        _out_dtype_code(out.dtype), out.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return out


def transpose_tile16(t: NVFP4Tensor, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """W^T of a 16x16-tile packed tensor, exactly (codes and scales moved, none re-quantized)."""
    if t.block != TILE16:
        raise ValueError("transpose_tile16 needs a TILE16 tensor")
    _need_gpu(t.codes)
    _check_packed(t, t.rows, t.cols, TILE16, "t")
    if out is None:
        out = empty_packed(t.cols, t.rows, TILE16, t.codes.device)
    _check_packed(out, t.cols, t.rows, TILE16, "out")
    _need_gpu(t.scales, t.alpha, out.codes, out.scales, out.alpha)
    _check("nvfp4_transpose_tile16", lib.nvfp4_transpose_tile16(
        _ptr(t.codes), _ptr(t.scales), _ptr(t.alpha), t.rows, t.cols, _ptr(out.codes), _ptr(out.scales),
        _ptr(out.alpha), _stream()))
    return out


def dgrad(dy: torch.Tensor, w_t: NVFP4Tensor, out_dtype=torch.bfloat16, rule="4over6",
          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """DGRAD dX = quantize(dY) @ W with w_t = transpose_tile16(W): the fused
    linear against the transposed weight (dY quantized in 16-blocks along the
    layer's output features, its contraction dimension)."""
    return linear(dy, w_t, out_dtype, rule, out=out, workspace=workspace)


def quantize_col16_rht(x: torch.Tensor, signs: int, rule="4over6", amax: torch.Tensor | None = None,
                       out: NVFP4Tensor | None = None, workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """COL16 quantization of the tensor after the 16-point random Hadamard
    transform of every column block (signs: 16-bit mask of the diagonal)."""
    _need_gpu(x, amax)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2D with unit column stride")
    rows, cols = x.shape
    _check_vec(amax, 1, torch.float32, "amax")
    if out is None:
        out = empty_packed(rows, cols, COL16, x.device)
    _check_packed(out, rows, cols, COL16, "out")
    if workspace is None and amax is None:
        workspace = torch.empty(lib.nvfp4_quantize_workspace_size(rows, cols), dtype=torch.uint8, device=x.device)
    _need_gpu(out.codes, out.scales, out.alpha, workspace)
    _check("nvfp4_quantize_col16_rht", lib.nvfp4_quantize_col16_rht(
        _ptr(x), _dtype_code(x), rows, cols, x.stride(0), _rule(rule), int(signs), _ptr(amax), _ptr(out.codes),
        _ptr(out.scales), _ptr(out.alpha), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream()))
    return out


class KvChunked:
    """KV tensors [*lead, heads, tokens, head_dim] (lead = () for one tensor,
    (tensors,) for several, e.g. a layer's K and V) packed with one global
    scale per tensor and chunk of tokens: codes [*lead, heads, tokens, d/2],
    scales [*lead, heads, tokens, d/16] (uint8), alphas [*lead, n_chunks]
    (float32)."""

    def __init__(self, codes, scales, alphas, heads, tokens, head_dim, tokens_per_chunk, lead=()):
        self.codes, self.scales, self.alphas = codes, scales, alphas
        self.heads, self.tokens, self.head_dim, self.tokens_per_chunk = heads, tokens, head_dim, tokens_per_chunk
        self.lead = tuple(lead)

    @property
    def tensors(self) -> int:
        return self.lead[0] if self.lead else 1


def kv_quantize_chunked(kv: torch.Tensor, tokens_per_chunk: int, rule="4over6",
                        out: KvChunked | None = None, chunk_amax: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> KvChunked:
    """quantize_kv with the pages' per-chunk global scale: kv [heads, tokens,
    head_dim] or [tensors, heads, tokens, head_dim] contiguous; chunk c of a
    tensor = tokens [c*tpc, (c+1)*tpc) of its every head.  chunk_amax
    (float32 [tensors * n_chunks], optional): the units' max |x|."""
    _need_gpu(kv)
    if kv.dim() not in (3, 4) or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [(tensors,) heads, tokens, head_dim] tensor")
    lead = tuple(kv.shape[:-3])
    tensors = lead[0] if lead else 1
    heads, tokens, d = kv.shape[-3:]
    tpc = int(tokens_per_chunk)
    nch = (tokens + tpc - 1) // tpc if tpc > 0 else 0
    if out is None:
        dev = kv.device
        out = KvChunked(torch.empty(lead + (heads, tokens, d // 2), dtype=torch.uint8, device=dev),
                        torch.empty(lead + (heads, tokens, d // 16), dtype=torch.uint8, device=dev),
                        torch.empty(lead + (max(nch, 1),), dtype=torch.float32, device=dev),
                        heads, tokens, d, tpc, lead)
    if (tuple(out.codes.shape) != lead + (heads, tokens, d // 2) or
            tuple(out.scales.shape) != lead + (heads, tokens, d // 16)):
        raise ValueError("output packed tensor has the wrong shape")
    for t, what in ((out.codes, "codes"), (out.scales, "scales")):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous uint8")
    _check_vec(out.alphas, tensors * nch, torch.float32, "alphas")
    _check_vec(chunk_amax, tensors * nch, torch.float32, "chunk_amax")
    if workspace is None:
        workspace = torch.empty(lib.nvfp4_kv_chunked_workspace_size(tensors, heads, tokens, d, tpc),
                                dtype=torch.uint8, device=kv.device)
    _need_gpu(out.codes, out.scales, out.alphas, chunk_amax, workspace)
    _check("nvfp4_kv_quantize_chunked", lib.nvfp4_kv_quantize_chunked(
        _ptr(kv), _dtype_code(kv), tensors, heads, tokens, d, tpc, _rule(rule), _ptr(chunk_amax),
        _ptr(out.codes), _ptr(out.scales), _ptr(out.alphas), _ptr(workspace), workspace.numel(), _stream()))
    return out


def kv_dequantize_chunked(t: KvChunked, dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """(q * s) * alpha of each element's tensor and chunk, [*lead, heads,
    tokens, head_dim]."""
    _need_gpu(t.codes, t.scales, t.alphas)
    shape = t.lead + (t.heads, t.tokens, t.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=t.codes.device)
    if tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the packed tensor's shape")
    _need_gpu(out)
    _check("nvfp4_kv_dequantize_chunked", lib.nvfp4_kv_dequantize_chunked(
        _ptr(t.codes), _ptr(t.scales), _ptr(t.alphas), t.tensors, t.heads, t.tokens, t.head_dim,
        t.tokens_per_chunk, _ptr(out), _out_dtype_code(out.dtype), _stream()))
    return out


def kv_quantize_smoothed(k: torch.Tensor, rule="4over6", out: NVFP4Tensor | None = None,
                         means: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Key smoothing (each key vector minus its mean over head_dim), then the
    KV quantizer; returns (packed keys, fp32 means [vectors])."""
    _need_gpu(k)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    d = k.shape[-1]
    v = k.numel() // d
    if out is None:
        out = empty_packed(v, d, ROW16, k.device)
    _check_packed(out, v, d, ROW16, "out")
    if means is None:
        means = torch.empty(v, dtype=torch.float32, device=k.device)
    _check_vec(means, v, torch.float32, "means")
    if workspace is None:
        workspace = torch.empty(lib.nvfp4_kv_smooth_workspace_size(v, d), dtype=torch.uint8, device=k.device)
    _need_gpu(out.codes, out.scales, out.alpha, means, workspace)
    _check("nvfp4_kv_quantize_smoothed", lib.nvfp4_kv_quantize_smoothed(
        _ptr(k), _dtype_code(k), v, d, _rule(rule), _ptr(out.codes), _ptr(out.scales), _ptr(out.alpha),
        _ptr(means), _ptr(workspace), workspace.numel(), _stream()))
    return out, means


def kv_dequantize_window(parts, out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rebuild an attention window in one launch.  parts: sequence of
    (packed chunk, means or None, first row, row count); rows are written in
    that order."""
    parts = list(parts)
    if len(parts) > MAX_KV_SEGMENTS:
        raise ValueError(f"at most {MAX_KV_SEGMENTS} segments")
    if not parts:
        raise ValueError("no segments")
    d = parts[0][0].cols
    rows = sum(int(c) for _, _, _, c in parts)
    segs = (KvSegment * len(parts))()
    for i, (t, means, first, count) in enumerate(parts):
        if t.block != ROW16 or t.cols != d:
            raise ValueError("segments must be ROW16 chunks of one head_dim")
        _check_packed(t, t.rows, d, ROW16, f"segment {i}")
        _check_vec(means, t.rows, torch.float32, f"segment {i} means")
        if first < 0 or count < 0 or first + count > t.rows:
            raise ValueError("segment rows out of range")
        _need_gpu(t.codes, t.scales, t.alpha, means)
        segs[i] = KvSegment(_ptr(t.codes), _ptr(t.scales), _ptr(t.alpha), _ptr(means), int(first), int(count))
    if out is None:
        out = torch.empty((rows, d), dtype=out_dtype, device=parts[0][0].codes.device)
    _check_out(out, (rows, d))
    _need_gpu(out)
    _check("nvfp4_kv_dequantize_window", lib.nvfp4_kv_dequantize_window(
        segs, len(parts), d, _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _stream()))
    return out


def kv_window_plan(frame: int, chunk_frames: int, window_frames: int, global_sink_frames: int = 0,
                   shot_start: int | None = None, shot_frames: int = 0):
    """Frames the attention of the chunk starting at `frame` reads, as
    (chunk index, first frame inside the chunk, frame count) runs in frame
    order: the global sink (frames [0, global_sink_frames)), the shot sink
    (frames [shot_start, shot_start + shot_frames)) and the sliding window
    (the window_frames frames before `frame`), each frame once.  Only frames
    before `frame` exist in the cache."""
    ranges = [(max(0, frame - window_frames), frame), (0, min(global_sink_frames, frame))]
    if shot_start is not None and shot_frames > 0:
        ranges.append((shot_start, min(shot_start + shot_frames, frame)))
    ranges = sorted((a, b) for a, b in ranges if b > a)
    merged = []
    for a, b in ranges:
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], b))
        else:
            merged.append((a, b))
    runs = []
    for a, b in merged:
        f = a
        while f < b:
            c = f // chunk_frames
            e = min(b, (c + 1) * chunk_frames)
            runs.append((c, f - c * chunk_frames, e - f))
            f = e
    return runs


def linear_lora(x: torch.Tensor, w: NVFP4Tensor, lora_a: torch.Tensor, lora_b: torch.Tensor, lora_scale: float,
                out_dtype=torch.bfloat16, rule="4over6", out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, u: torch.Tensor | None = None, amax_out=None):
    """W4A4 linear plus the BF16 LoRA branch: y = quantize(x) @ w^T +
    lora_scale * bf16(x @ lora_a^T) @ lora_b^T.  Returns (y, U)."""
    _need_gpu(x, lora_a, lora_b)
    if x.dtype != torch.bfloat16 or lora_a.dtype != torch.bfloat16 or lora_b.dtype != torch.bfloat16:
        raise TypeError("the LoRA path takes bf16 x, lora_a and lora_b")
    if x.dim() != 2 or x.stride(1) != 1 or not lora_a.is_contiguous() or not lora_b.is_contiguous():
        raise ValueError("x 2D with unit column stride; lora_a, lora_b contiguous")
    cw, sw, aw, lw, n, kw = w.operand()
    m, k = x.shape
    r = lora_a.shape[0]
    if k != kw or lora_a.shape[1] != k or tuple(lora_b.shape) != (n, r):
        raise ValueError("shape mismatch")
    _check_packed(w, w.rows, w.cols, w.block, "w")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check_out(out, (m, n))
    if u is None:
        u = torch.empty((m, r), dtype=torch.bfloat16, device=x.device)
    if tuple(u.shape) != (m, r) or u.dtype != torch.bfloat16 or not u.is_contiguous():
        raise ValueError(f"u must be a contiguous bfloat16 [{m}, {r}] tensor")
    _check_vec(amax_out, 1, torch.float32, "amax_out")
    if workspace is None:
        workspace = torch.empty(lib.nvfp4_linear_lora_workspace_size(m, k, r), dtype=torch.uint8, device=x.device)
    _need_gpu(cw, sw, aw, u, out, amax_out, workspace)
    _check("nvfp4_linear_lora", lib.nvfp4_linear_lora(
        _ptr(x), m, k, x.stride(0), _rule(rule), _ptr(cw), _ptr(sw), _ptr(aw), lw, n, _ptr(lora_a), _ptr(lora_b), r,
        float(lora_scale), _ptr(u), _ptr(out), _out_dtype_code(out.dtype), out.stride(0), _ptr(amax_out),
        _ptr(workspace), workspace.numel(), _stream()))
    return out, u
