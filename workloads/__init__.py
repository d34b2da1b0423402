"""Seeded synthetic inputs for the E8-codebook linear layer.

This module only draws random numbers. It holds none of the method's
arithmetic (no codebook, no Hadamard transform, no scale rule, no
quantisation): both the oracle-based tests and the GPU path take their
inputs from here, so it must stay independent of either side.

Layer shapes and distributions follow the five synthetic layer workloads
the library is measured on (an E8 lattice codebook, "glq 0.1.1", section
"How it works", and the EntroPack news item's framing of fused runtime
weight reconstruction):

  small       256x256,   2 bpw, M=4,    W ~ N(0, 0.02),       x fp32 N(0,1)
  gemv        4096x4096, 2 bpw, M=1,    W ~ Student-t(5) std 0.02,
                                        x bf16 N(0,1), 8 outlier channels x20
  batch16     4096x4096, 4 bpw, M=16,   W ~ N(0, 0.02),       x bf16 N(0,1)
  prefill_up  16384x4096,3 bpw, M=2048, W ~ Student-t(5) std 0.02,
                                        x bf16 N(0,1), 1% outlier channels x20
  dit_block   Q,K,V,O 3072x3072, up 12288x3072, down 3072x12288,
              4 bpw, M=4096, W ~ N(0, 0.02), x bf16 N(0,1) per linear

Seeds: workload number c (1..5) uses base = 1000*c; the streams are
W = base+0, x = base+1, sign_k = base+2, sign_n = base+3, outlier
channels = base+4, calibration inputs = base+5 (for the DiT block, linear
number l adds 100*l).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerSpec", "WORKLOADS", "layer_specs", "weights", "activations",
    "signs", "random_indices", "bf16_round_trip", "calibration",
]


@dataclass(frozen=True)
class LayerSpec:
    name: str
    n: int                 # out features
    k: int                 # in features
    bpw: int               # 2, 3 or 4
    m: int                 # activation rows (tokens)
    w_dist: str            # "normal" | "student_t"
    x_dtype: str           # "f32" | "bf16"
    y_dtype: str           # "f32" | "bf16"
    outliers: int = 0      # number of outlier activation channels (x20)
    seed_base: int = 0
    meta: dict = field(default_factory=dict, compare=False)


def _dit_block():
    shapes = [("q", 3072, 3072), ("k", 3072, 3072), ("v", 3072, 3072),
              ("o", 3072, 3072), ("up", 12288, 3072), ("down", 3072, 12288)]
    return tuple(
        LayerSpec(f"dit_block.{nm}", n, k, 4, 4096, "normal", "bf16", "bf16",
                  0, 5000 + 100 * i)
        for i, (nm, n, k) in enumerate(shapes))


WORKLOADS = {
    "small": (LayerSpec("small", 256, 256, 2, 4, "normal", "f32", "f32", 0, 1000),),
    "gemv": (LayerSpec("gemv", 4096, 4096, 2, 1, "student_t", "bf16", "bf16", 8, 2000),),
    "batch16": (LayerSpec("batch16", 4096, 4096, 4, 16, "normal", "bf16", "bf16", 0, 3000),),
    "prefill_up": (LayerSpec("prefill_up", 16384, 4096, 3, 2048, "student_t", "bf16",
                             "bf16", round(0.01 * 4096), 4000),),
    "dit_block": _dit_block(),
}


def layer_specs(workload: str):
    return WORKLOADS[workload]


def weights(spec: LayerSpec, rows=None) -> np.ndarray:
    """W [n, k] float64 in the original (unrotated) basis.

    Student-t(5) draws are divided by sqrt(5/3), the standard deviation of a
    unit Student-t with 5 degrees of freedom, so the std is 0.02.
    `rows` (a slice) returns only those rows, drawn from the same stream.
    """
    rng = np.random.default_rng(spec.seed_base + 0)
    if spec.w_dist == "normal":
        w = rng.normal(0.0, 0.02, size=(spec.n, spec.k))
    elif spec.w_dist == "student_t":
        w = rng.standard_t(5, size=(spec.n, spec.k)) * (0.02 / math.sqrt(5.0 / 3.0))
    else:
        raise ValueError(spec.w_dist)
    return w if rows is None else w[rows]


def activations(spec: LayerSpec, m: int | None = None) -> np.ndarray:
    """x [m, k] float32: N(0,1), with `outliers` channels scaled by 20.

    For bf16 workloads the caller rounds to bf16 (bf16_round_trip) so both
    sides see identical values.
    """
    m = spec.m if m is None else m
    rng = np.random.default_rng(spec.seed_base + 1)
    x = rng.standard_normal(size=(m, spec.k)).astype(np.float32)
    if spec.outliers:
        ch = np.random.default_rng(spec.seed_base + 4).choice(
            spec.k, spec.outliers, replace=False)
        x[:, ch] *= np.float32(20.0)
    if spec.x_dtype == "bf16":
        x = bf16_round_trip(x)
    return x


def signs(n: int, seed: int) -> np.ndarray:
    """+-1 sign vector (int8) of length n from a PCG64 stream."""
    b = np.random.default_rng(seed).integers(0, 2, size=n)
    return (1 - 2 * b).astype(np.int8)


def sign_k(spec: LayerSpec) -> np.ndarray:
    return signs(spec.k, spec.seed_base + 2)


def sign_n(spec: LayerSpec) -> np.ndarray:
    return signs(spec.n, spec.seed_base + 3)


def calibration(spec: LayerSpec, m: int, rho: float = 0.6) -> np.ndarray:
    """Calibration inputs X [m, k] float64 for a synthetic Hessian X^T X / m.

    Unit normals made first-order autoregressive along k (neighbouring input
    channels correlated with coefficient rho, unit variance kept), with the
    same outlier channels as activations() scaled by 20. Stream base+5.
    """
    rng = np.random.default_rng(spec.seed_base + 5)
    z = rng.standard_normal(size=(m, spec.k))
    x = np.empty_like(z)
    x[:, 0] = z[:, 0]
    c = math.sqrt(1.0 - rho * rho)
    for j in range(1, spec.k):
        x[:, j] = rho * x[:, j - 1] + c * z[:, j]
    if spec.outliers:
        ch = np.random.default_rng(spec.seed_base + 4).choice(
            spec.k, spec.outliers, replace=False)
        x[:, ch] *= 20.0
    return x


def random_indices(shape, seed: int, upper: int = 65536, dtype=np.uint16) -> np.ndarray:
    """Uniform random codebook indices (for shape/edge-case tests at sizes
    where running the nearest-neighbour encoder would be too slow)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, upper, size=shape).astype(dtype)


def bf16_round_trip(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32. Plain IEEE rounding of the input, not part of the method."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
