"""Seeded synthetic inputs for the NVFP4 W4A4 linear layer and the NVFP4 KV cache.

This module only draws random tensors. It holds none of the quantizer's or the
GEMM's arithmetic, so both the CPU oracle and the HIP path can take their
inputs from here without sharing any of the method.

Shapes follow the 5B video DiT the pages describe ("LongLive-2.0: An NVFP4
Parallel Infrastructure for Long Video Generation", paper notes page, section
3.6/4 inference setup): 24 heads x head_dim 128 = hidden 3072, and 880 latent
tokens per frame ((44/2) x (80/2) patches of a 44x80 latent).  The pages train
and evaluate on real videos and trained weights, which are not available;
these tensors stand in for them.

Recipe (every config):
  * generator: numpy.random.Generator(PCG64(seed));
  * normals are drawn in float64, multiplied by sigma, cast to float32, then
    to bfloat16 by round-to-nearest-even when the config is bf16;
  * outliers: exactly round(0.001 * numel) distinct positions (choice without
    replacement) are multiplied by 50 before the bf16 cast;
  * draw order inside a config: X, then W, then the third tensor.

bf16 tensors are returned as numpy uint16 arrays of raw bit patterns (numpy
has no bfloat16); `bf16_to_f32` widens them exactly.
"""
from __future__ import annotations

import numpy as np

SEEDS = {1: 0, 2: 2, 3: 3, 4: 4, 5: 5}

# DiT geometry
HEADS = 24
HEAD_DIM = 128
HIDDEN = HEADS * HEAD_DIM          # 3072
TOKENS_PER_FRAME = 880             # (44/2) * (80/2)
FFN = 14336


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(g: np.random.Generator, shape, sigma: float, outlier_frac: float = 0.0,
               outlier_gain: float = 50.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float64) * sigma
    if outlier_frac > 0.0:
        n = int(round(outlier_frac * x.size))
        pos = g.choice(x.size, size=n, replace=False)
        x.reshape(-1)[pos] *= outlier_gain
    return x.astype(np.float32)


def normal_bf16(g, shape, sigma, outlier_frac=0.0):
    return f32_to_bf16_bits(normal_f32(g, shape, sigma, outlier_frac))


def config1(seed: int = SEEDS[1]):
    """Tiny linear: X fp32 [64,128] ~ N(0,1), W fp32 [64,128] ~ N(0,0.02)."""
    g = rng(seed)
    x = normal_f32(g, (64, 128), 1.0)
    w = normal_f32(g, (64, 128), 0.02)
    return {"x": x, "w": w}


def config2(seed: int = SEEDS[2], m: int = 3 * TOKENS_PER_FRAME, k: int = HIDDEN,
            n: int = 3 * HIDDEN):
    """QKV projection: X bf16 [2640,3072] N(0,1) + 0.1% x50; W bf16 [9216,3072] N(0,0.02)."""
    g = rng(seed)
    x = normal_bf16(g, (m, k), 1.0, 0.001)
    w = normal_bf16(g, (n, k), 0.02)
    return {"x": x, "w": w}


def config3(seed: int = SEEDS[3], m: int = 3 * TOKENS_PER_FRAME, k: int = HIDDEN,
            f: int = FFN):
    """FFN pair: up X [2640,3072] x W_up [14336,3072]^T; down A=|N(0,1)|^1.5 [2640,14336] x W_down [3072,14336]^T."""
    g = rng(seed)
    x = normal_bf16(g, (m, k), 1.0, 0.001)
    w_up = normal_bf16(g, (f, k), 0.02)
    a = np.abs(g.standard_normal(size=(m, f), dtype=np.float64)) ** 1.5
    a = f32_to_bf16_bits(a.astype(np.float32))
    w_down = normal_bf16(g, (k, f), 0.02)
    return {"x": x, "w_up": w_up, "a": a, "w_down": w_down}


def config4(seed: int = SEEDS[4], heads: int = HEADS, tokens: int = 21 * TOKENS_PER_FRAME,
            head_dim: int = HEAD_DIM):
    """KV cache: K, V bf16 [24, 18480, 128] = N(0,1) * c[h,d], log10 c ~ U[-1,1].

    One channel factor per (head, head_dim channel), shared by all tokens;
    K and V get independent draws (K's factor, K, V's factor, V).
    """
    g = rng(seed)
    out = {}
    for name in ("k", "v"):
        c = 10.0 ** g.uniform(-1.0, 1.0, size=(heads, 1, head_dim))
        t = g.standard_normal(size=(heads, tokens, head_dim), dtype=np.float64) * c
        out[name] = f32_to_bf16_bits(t.astype(np.float32))
    return out


def config5(seed: int = SEEDS[5], m: int = 32768, k: int = HIDDEN, n: int = HIDDEN):
    """Training linear: X bf16 [32768,3072] + 0.1% x50; W [3072,3072] N(0,0.02); dY [32768,3072] N(0,1e-3)."""
    g = rng(seed)
    x = normal_bf16(g, (m, k), 1.0, 0.001)
    w = normal_bf16(g, (n, k), 0.02)
    dy = normal_bf16(g, (m, n), 1e-3)
    return {"x": x, "w": w, "dy": dy}


def random_bf16(seed: int, shape, sigma: float = 1.0, outlier_frac: float = 0.0):
    """Generic seeded bf16 tensor for shape sweeps (ragged sizes, edge cases)."""
    return normal_bf16(rng(seed), shape, sigma, outlier_frac)
