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


def lora_u_window(x: np.ndarray, la: np.ndarray):
    """For U = x A^T summed in fp32 and rounded once to bf16: the bf16 bits
    at the two ends of the window a correct kernel can land in.

    The kernel's fp32 sum s obeys |s - exact| <= B with
      B = K * 2^-24 * sum|x a|     (recursive fp32 summation of K products)
        + K * 2^-126               (the matrix cores flush subnormal fp32
                                    products and partial sums to zero)
        + K * 2^-52 * sum|x a|     (the fp64 evaluation of `exact` here),
    and bf16 rounding is monotone, so a correct U lies between
    RNE_bf16(exact - B) and RNE_bf16(exact + B).  Where those two agree the
    window is a single value: the oracle's rounding of the exact sum."""
    xf = workloads.bf16_to_f32(x).astype(np.float64)
    af = workloads.bf16_to_f32(la).astype(np.float64)
    exact = xf @ af.T
    k = xf.shape[1]
    mag = np.abs(xf) @ np.abs(af).T
    bound = k * (2.0 ** -24 + 2.0 ** -52) * mag + k * 2.0 ** -126
    return oracle.bf16_rne_f64(exact - bound), oracle.bf16_rne_f64(exact + bound)


def check_lora_u(ug: np.ndarray, x: np.ndarray, la: np.ndarray) -> int:
    """U from the kernel equals the oracle's U (the exact sum rounded once to
    bf16, oracle.lora_down_bf16) except where the exact sum lies within the
    fp32 accumulation bound of a bf16 rounding boundary; there, U must be one
    of the bf16 values inside that window (lora_u_window).  Returns the
    number of elements that differ from the oracle's U."""
    lo, hi = lora_u_window(x, la)
    u = workloads.bf16_to_f32(ug)
    flo, fhi = workloads.bf16_to_f32(lo), workloads.bf16_to_f32(hi)
    outside = (u < flo) | (u > fhi)
    if np.any(outside):
        i = tuple(np.argwhere(outside)[0])
        raise AssertionError(f"U outside its accumulation window at {i}: {u[i]} not in [{flo[i]}, {fhi[i]}]")
    uref = oracle.lora_down_bf16(x, la)
    single = lo == hi
    bad = single & (ug != uref)
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"U differs from the oracle's rounding at {i} away from any boundary: "
                             f"{ug[i]:#06x} vs {uref[i]:#06x}")
    return int(np.count_nonzero(ug != uref))


def lora_branch_allowance(ug: np.ndarray, uref: np.ndarray, lb: np.ndarray, scale: float, ms=None, ns=None):
    """|scale| * sum_r |U - Uref|[m, r] |B|[n, r]: how far y may move because
    the kernel's U differs from the oracle's U (only at rounding windows);
    zero on rows where the two agree.  ms/ns: sampled positions (else all)."""
    du = np.abs(workloads.bf16_to_f32(ug).astype(np.float64) - workloads.bf16_to_f32(uref).astype(np.float64))
    bb = np.abs(workloads.bf16_to_f32(lb).astype(np.float64))
    if ms is None:
        return abs(scale) * (du @ bb.T)
    return abs(scale) * np.einsum("ij,ij->i", du[ms], bb[ns])


def check_y_on_oracle_u(got: np.ndarray, ref_oracle_u: np.ndarray, allow: np.ndarray):
    """y against the fp64 reference built entirely by the oracle (activation
    codes, weight codes and U): what exceeds the allowance of the U rounding
    windows must stay within the relative Frobenius bound."""
    excess = np.maximum(np.abs(got.astype(np.float64) - ref_oracle_u) - allow, 0.0)
    den = np.linalg.norm(ref_oracle_u)
    if den == 0.0:
        assert not np.any(excess), "nonzero output where the oracle's is zero"
        return 0.0
    err = float(np.linalg.norm(excess) / den)
    assert err <= GEMM_RTOL, err
    return err
