"""Seeded synthetic inputs for the tiled half-precision GEMM.

This module only draws random numbers and rounds them to the 16-bit storage
formats; it holds none of the GEMM's arithmetic.  Both sides of every parity
check (the CPU oracle and the HIP path) take their operands from here, as raw
16-bit patterns (numpy ``uint16``), so that they start from the same bits.

Workloads are the five shapes the tiled GEMM is measured on: a small square
case, a 4096-cube, a bf16 shape whose sides are no multiple of any tile, a
decode-shaped skinny product (M=16) and an 8192-cube with the fused bias +
GELU(tanh) epilogue.  Distributions, seeds and the sampled-row recipe for the
largest shape are fixed here and nowhere else.

Recipe: ``numpy.random.Generator(PCG64(seed))`` draws float32 values, which are
rounded to fp16 by numpy's float32->float16 cast and to bf16 by torch's
float32->bfloat16 cast (both round to nearest, ties to even).  For workload
number i (1..5) the seeds are A = 1000*i+1, B = 1000*i+2, bias = 1000*i+3 and
sampled rows = 1000*i+4.  "uniform[lo,hi]" draws ``lo + (hi-lo)*U[0,1)``;
"normal(mu, sigma)" reads sigma as a standard deviation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# Storage formats and epilogues, numbered as in the C interface (tg_gemm.h).
F16 = 0
BF16 = 1
EPI_NONE = 0
EPI_BIAS = 1
EPI_BIAS_GELU_TANH = 2

DTYPE_NAMES = {F16: "f16", BF16: "bf16"}
EPI_NAMES = {EPI_NONE: "none", EPI_BIAS: "bias", EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}

Dist = Tuple[str, float, float]  # ("uniform", lo, hi) or ("normal", mean, std)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # 1..5; fixes the seeds
    M: int
    N: int
    K: int
    dtype: int
    epilogue: int
    a_dist: Dist
    b_dist: Dist
    bias_dist: Optional[Dist]
    sampled_rows: Optional[int]   # None: the oracle checks every row

    @property
    def seeds(self):
        b = 1000 * self.index
        return {"A": b + 1, "B": b + 2, "bias": b + 3, "rows": b + 4}


WORKLOADS = {
    w.name: w
    for w in [
        Workload("gemm_f16_256x256x256", 1, 256, 256, 256, F16, EPI_NONE,
                 ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), None, None),
        Workload("gemm_f16_4096x4096x4096", 2, 4096, 4096, 4096, F16, EPI_NONE,
                 ("normal", 0.0, 0.1), ("normal", 0.0, 0.1), None, 64),
        Workload("gemm_bf16_4000x4093x4111_bias_gelu_tanh", 3, 4000, 4093, 4111, BF16,
                 EPI_BIAS_GELU_TANH, ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0),
                 ("uniform", -0.5, 0.5), 64),
        Workload("gemm_f16_skinny_16x11008x4096", 4, 16, 11008, 4096, F16, EPI_NONE,
                 ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), None, None),
        Workload("gemm_f16_8192x8192x8192_bias_gelu_tanh", 5, 8192, 8192, 8192, F16,
                 EPI_BIAS_GELU_TANH, ("normal", 0.0, 0.05), ("normal", 0.0, 0.05),
                 ("normal", 0.0, 0.1), 64),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)

# Shape classes for the choice of tile size: outputs with few 256 x 256 tiles
# next to the ones above.  The pages' own GEMM benchmark shape (a 2048-cube),
# a batch of 512 rows through the decode shape's 11008-wide weight, a small
# output with a deep K, and a ragged mid-size bf16 shape with the epilogue.
# Same recipe, with workload numbers 11.. for the seeds.
TILE_WORKLOADS = {
    w.name: w
    for w in [
        Workload("gemm_f16_2048x2048x2048", 11, 2048, 2048, 2048, F16, EPI_NONE,
                 ("normal", 0.0, 0.1), ("normal", 0.0, 0.1), None, 64),
        Workload("gemm_f16_512x11008x4096", 12, 512, 11008, 4096, F16, EPI_NONE,
                 ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), None, 64),
        Workload("gemm_f16_1024x1024x8192", 13, 1024, 1024, 8192, F16, EPI_NONE,
                 ("normal", 0.0, 0.1), ("normal", 0.0, 0.1), None, 64),
        Workload("gemm_bf16_1000x3000x6000_bias_gelu_tanh", 14, 1000, 3000, 6000, BF16,
                 EPI_BIAS_GELU_TANH, ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0),
                 ("uniform", -0.5, 0.5), 64),
    ]
}


def _draw_f32(rng: np.random.Generator, shape, dist: Dist) -> np.ndarray:
    kind, p0, p1 = dist
    if kind == "uniform":
        u = rng.random(shape, dtype=np.float32)
        return (np.float32(p0) + np.float32(p1 - p0) * u).astype(np.float32)
    if kind == "normal":
        z = rng.standard_normal(shape, dtype=np.float32)
        return (np.float32(p0) + np.float32(p1) * z).astype(np.float32)
    raise ValueError(f"unknown distribution {kind!r}")


def round_f32(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 values to fp16/bf16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unknown dtype {dtype}")


def random_bits(shape, dist: Dist, dtype: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_f32(_draw_f32(rng, shape, dist), dtype)


def small_int_bits(shape, dtype: int, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi]; exact in both 16-bit formats."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return round_f32(v, dtype)


def values_bits(values: np.ndarray, dtype: int) -> np.ndarray:
    """Round arbitrary float values (via float32) to 16-bit patterns."""
    return round_f32(np.asarray(values, dtype=np.float32), dtype)


def sampled_rows(w: Workload) -> np.ndarray:
    """Rows the oracle checks: all rows, or {0, M-1} plus seeded distinct rows."""
    if w.sampled_rows is None or w.sampled_rows >= w.M:
        return np.arange(w.M, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(w.seeds["rows"]))
    inner = rng.choice(np.arange(1, w.M - 1), size=w.sampled_rows - 2, replace=False)
    return np.sort(np.concatenate([[0, w.M - 1], inner]).astype(np.int64))


@dataclass
class Operands:
    workload: Workload
    A: np.ndarray                # uint16 bits, (M, K) row-major
    B: np.ndarray                # uint16 bits, (K, N) row-major
    bias: Optional[np.ndarray]   # uint16 bits, (N,), or None
    rows: np.ndarray             # int64 rows the oracle checks


def make_operands(w: Workload) -> Operands:
    s = w.seeds
    A = random_bits((w.M, w.K), w.a_dist, w.dtype, s["A"])
    B = random_bits((w.K, w.N), w.b_dist, w.dtype, s["B"])
    bias = None
    if w.epilogue != EPI_NONE:
        bias = random_bits((w.N,), w.bias_dist, w.dtype, s["bias"])
    return Operands(w, A, B, bias, sampled_rows(w))


def make_small_int_operands(w: Workload, with_bias: bool = True) -> Operands:
    """Same shape as ``w`` but entries in {-2..2}: every fp32 partial sum is exact."""
    s = w.seeds
    A = small_int_bits((w.M, w.K), w.dtype, s["A"] + 500)
    B = small_int_bits((w.K, w.N), w.dtype, s["B"] + 500)
    bias = small_int_bits((w.N,), w.dtype, s["bias"] + 500) if (with_bias and w.epilogue != EPI_NONE) else None
    return Operands(w, A, B, bias, sampled_rows(w))


def w4_weights(K: int, N: int, seed: int) -> np.ndarray:
    """4-bit weight codes, uniform over 0..15, one per byte, (K, N)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 16, size=(K, N)).astype(np.uint8)


# The weight-only 4-bit product timed beside the 16-bit decode shape: the same
# M, N, K, with 128-row scale groups.
W4_WORKLOAD = dict(name="gemm_w4_f16_16x11008x4096_g128", M=16, N=11008, K=4096, group=128, dtype=F16,
                   a_dist=("normal", 0.0, 1.0), scale_dist=("uniform", 0.001, 0.01), seeds=(6001, 6002, 6003))


# The attention forward at the shape of the FlashAttention pages' benchmark:
# batch 1, 32 heads of width 128, 4096 queries and keys, standard-normal
# Q, K and V, timed without and with the causal mask.
ATTN_WORKLOAD = dict(name="attention_fwd_f16_b1_h32_s4096_d128", batch=1, heads=32, seq=4096, head_dim=128,
                     dtype=F16, dist=("normal", 0.0, 1.0), seeds=(7001, 7002, 7003))
