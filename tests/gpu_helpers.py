"""Shared helpers of the GPU parity tests: host<->device marshalling and the
comparison rules (bit-exact for codes/scales/alpha, relative Frobenius 1e-5
for fp32-accumulated GEMM outputs)."""
import numpy as np
import torch

import oracle
import workloads

GEMM_RTOL = 1e-5          # relative Frobenius bound on fp32 GEMM outputs


def dev_from_host(x: np.ndarray) -> torch.Tensor:
    """numpy fp32 array, or uint16 bf16 bit patterns, -> device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_packed_equal(gpu, ref: oracle.Packed, what=""):
    codes = gpu.codes.cpu().numpy()
    scales = gpu.scales.cpu().numpy()
    alpha = gpu.alpha.cpu().numpy()[0]
    assert alpha.view(np.uint32) == np.float32(ref.alpha).view(np.uint32), (what, alpha, ref.alpha)
    if not np.array_equal(scales, ref.scales):
        bad = np.argwhere(scales != ref.scales)
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first {bad[:5].tolist()} "
                             f"gpu {scales[tuple(bad[0])]} ref {ref.scales[tuple(bad[0])]}")
    if not np.array_equal(codes, ref.codes):
        bad = np.argwhere(codes != ref.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first {bad[:5].tolist()} "
                             f"gpu {codes[tuple(bad[0])]:#x} ref {ref.codes[tuple(bad[0])]:#x}")


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm(got.astype(np.float64) - ref.astype(np.float64))
    den = np.linalg.norm(ref.astype(np.float64))
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)


def packed_to_device(p: oracle.Packed):
    """An oracle-packed tensor as the binding's NVFP4Tensor (for GEMM inputs)."""
    import nvfp4_w4a4_quantized_04_amd as nv
    return nv.NVFP4Tensor(torch.from_numpy(p.codes.copy()).cuda(), torch.from_numpy(p.scales.copy()).cuda(),
                          torch.tensor([p.alpha], dtype=torch.float32).cuda(), p.rows, p.cols, p.block)


def check_lora_u(ug: np.ndarray, x: np.ndarray, la: np.ndarray):
    """U from the kernel is a correct bf16 rounding of a sum within the fp32
    accumulation bound of x A^T: |U - exact| <= half a bf16 step of U plus
    K * 2^-24 * sum |x a|, plus K * 2^-126 because the matrix cores flush fp32
    subnormal products and partial sums (below 2^-126) to zero; and, where the
    exact sum is far above that range, it equals the oracle's rounding of the
    exact sum except where the two sums straddle a rounding point (rare)."""
    xf = workloads.bf16_to_f32(x).astype(np.float64)
    af = workloads.bf16_to_f32(la).astype(np.float64)
    exact = xf @ af.T
    k = xf.shape[1]
    bound = k * 2.0 ** -24 * (np.abs(xf) @ np.abs(af).T)
    u = workloads.bf16_to_f32(ug).astype(np.float64)
    step = np.abs(u) * 2.0 ** -7                       # one bf16 step at |u| (or more)
    assert np.all(np.abs(u - exact) <= 0.5 * step + bound + k * 2.0 ** -126)
    uref = oracle.lora_down_bf16(x, la)
    normal = np.abs(exact) >= 2.0 ** -100
    if np.any(normal):
        assert np.mean(ug[normal] == uref[normal]) >= 0.99
