"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module holds no arithmetic of the method (no scaling, no FP8 encoding, no
GEMM).  It only draws random tensors and stores them in the input dtype,
bf16, as uint16 bit patterns.  The oracle and the HIP path both read the same
bytes it returns; nothing here is reproduced in another language.

Recipe (every tensor): ``np.random.default_rng(SeedSequence([workload,
tensor_id]))``; draw in float64; apply outliers / channel scaling; cast to
float32; round to bf16 with round-to-nearest-even on the bit pattern.
tensor_id: 0 = activation / A / dY, 1 = weight / B, 2 = optimizer-update noise,
3 = outlier positions or channel picks (A side), 4 = channel picks (B side).
"""
from __future__ import annotations

import numpy as np

# Workloads (shapes of the MLP up-projection of a 768-wide GPT at 64 x 1024
# tokens, and of a fine-grained block-scaled GEMM).
SMALL_UP_PROJ = dict(workload=1, x=(256, 768), w=(3072, 768))
QUANT_ONLY = dict(workload=2, x=(8192, 8192))
SPEEDRUN_UP_PROJ = dict(workload=3, x=(65536, 768), w=(3072, 768))
BLOCK_SCALED = dict(workload=4, a=(16384, 7168), b=(2048, 7168))
UP_PROJ_BACKWARD = dict(workload=5, dy=(65536, 3072))


def rng(workload: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(workload), int(tensor_id)]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return uint16 bits.
    NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16).astype(np.uint16)) | 0x0040
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(workload: int, tensor_id: int, shape, sigma: float, chunk: int = 1 << 24) -> np.ndarray:
    """bf16 N(0, sigma^2) tensor, drawn in float64 in chunks to bound memory."""
    g = rng(workload, tensor_id)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = g.standard_normal(e - s) * sigma
        out[s:e] = f32_to_bf16_bits(v.astype(np.float32))
    return out.reshape(shape)


def with_outliers_bf16(workload: int, shape, frac: float = 1e-3,
                       lo: float = 500.0, hi: float = 5000.0) -> np.ndarray:
    """N(0,1) with round(frac * N) distinct positions replaced by +-U(lo, hi).
    Positions are uniform without replacement; sign +-1 with probability 1/2."""
    g = rng(workload, 0)
    n = int(np.prod(shape))
    v = g.standard_normal(n)
    g3 = rng(workload, 3)
    count = int(round(frac * n))
    pos = g3.choice(n, size=count, replace=False)
    sign = np.where(g3.random(count) < 0.5, -1.0, 1.0)
    mag = g3.uniform(lo, hi, size=count)
    v[pos] = sign * mag
    return f32_to_bf16_bits(v.astype(np.float32)).reshape(shape)


def channel_scaled_bf16(workload: int, tensor_id: int, pick_id: int, shape,
                        frac: float = 0.01, factor: float = 100.0) -> np.ndarray:
    """N(0,1) with round(frac * K) distinct columns (the contiguous K channels)
    multiplied by `factor` before the bf16 rounding."""
    rows, cols = shape
    g = rng(workload, tensor_id)
    v = g.standard_normal((rows, cols))
    picks = rng(workload, pick_id).choice(cols, size=int(round(frac * cols)), replace=False)
    v[:, picks] *= factor
    return f32_to_bf16_bits(v.astype(np.float32))


def update_noise_f32(workload: int, shape, sigma: float = 1e-4) -> np.ndarray:
    """The optimizer update used to exercise the weight-cache refresh: fp32
    N(0, sigma^2) noise."""
    return (rng(workload, 2).standard_normal(shape) * sigma).astype(np.float32)


def apply_update_bf16(w_bits: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """W <- bf16(fp32(W) + noise): the master stays bf16, the add is fp32."""
    return f32_to_bf16_bits(bf16_bits_to_f32(w_bits) + noise.astype(np.float32))


def all_bf16_patterns() -> np.ndarray:
    """Every one of the 65,536 bf16 bit patterns, as a [256, 256] tensor."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)


def small_shape_bf16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """Generic seeded bf16 tensor for tiny / ragged test shapes (workload id 100+)."""
    return normal_bf16(100 + int(seed), 0, shape, sigma)
