"""Seeded synthetic inputs for the streaming log-domain Sinkhorn workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no arithmetic of the method itself: it only draws point clouds,
weights and value matrices, rounds them to their storage format, and decodes
stored bf16 bit patterns back to floating point.

The FlashSinkhorn pages describe their point-cloud workloads only as
n in [5k, 50k] and d in [4, 1024] (replication report, "Strengths" and
"Reproducibility" paragraphs); these generators stand in for them.

Seeding: ``numpy.random.default_rng([config_id, stream])`` with one stream per
array (x=0, y=1, a=2, b=3, V=4, U=5), so every array is reproducible on its own,
at any shape.
Rounding: values are drawn in float64, rounded to float32 (round to nearest
even), and for bf16 storage rounded again from float32 to bf16 (RNE).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

STREAM_X, STREAM_Y, STREAM_A, STREAM_B, STREAM_V, STREAM_U = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    """One workload: shapes, storage dtype, distributions and schedule."""
    cid: int                 # seed id
    name: str
    n: int
    m: int
    d: int
    dtype: str               # "f32" or "bf16": storage of x and y
    points: str              # "unit_vs_gauss" | "mixture8" | "gauss_over_sqrt_d"
    weights: str             # "uniform" | "dirichlet1"
    eps: float
    iters: int
    mode: str                # "alternating" | "symmetric"
    grad: bool = False       # barycentric gradient w.r.t. x after the solve
    apply_k: int = 0         # width of V and U for P.V and P^T.U (0: none)

    def scaled(self, n: int, m: Optional[int] = None, iters: Optional[int] = None) -> "Workload":
        """Same distributions and parameters at a smaller shape (for parity tests)."""
        return replace(self, n=n, m=n if m is None else m,
                       iters=self.iters if iters is None else iters)


# The five point-cloud configurations, the n=m=50k d=3 shape (key 6) and the bf16
# variant of the d=512 configuration (key 7, same seed and points as key 4).
CASES = {
    1: Workload(1, "tiny_d3", 1024, 1024, 3, "f32", "unit_vs_gauss", "uniform", 0.05, 50, "alternating"),
    2: Workload(2, "mix8_d3_10k", 10_000, 10_000, 3, "f32", "mixture8", "uniform", 0.01, 100, "symmetric", grad=True),
    3: Workload(3, "embed_d64_50k_bf16", 50_000, 50_000, 64, "bf16", "gauss_over_sqrt_d", "dirichlet1", 0.1, 100, "alternating"),
    4: Workload(4, "hidim_d512_20k", 20_000, 20_000, 512, "f32", "gauss_over_sqrt_d", "uniform", 0.5, 50, "alternating", grad=True),
    5: Workload(5, "rect_d1024_5k_50k_bf16", 5_000, 50_000, 1024, "bf16", "gauss_over_sqrt_d", "uniform", 1.0, 30, "alternating", apply_k=16),
    6: Workload(6, "mix8_d3_50k", 50_000, 50_000, 3, "f32", "mixture8", "uniform", 0.01, 100, "alternating"),
    7: Workload(4, "hidim_d512_20k_bf16", 20_000, 20_000, 512, "bf16", "gauss_over_sqrt_d", "uniform", 0.5, 50, "alternating", grad=True),
}


def _rng(cid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cid, stream])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _points(w: Workload, stream: int, count: int) -> np.ndarray:
    rng = _rng(w.cid, stream)
    if w.points == "unit_vs_gauss":
        if stream == STREAM_X:
            p = rng.uniform(0.0, 1.0, size=(count, w.d))
        else:
            p = 0.5 + 0.2 * rng.standard_normal((count, w.d))
    elif w.points == "mixture8":
        means = rng.uniform(0.0, 1.0, size=(8, w.d))
        labels = rng.integers(0, 8, size=count)
        p = means[labels] + 0.05 * rng.standard_normal((count, w.d))
    elif w.points == "gauss_over_sqrt_d":
        p = rng.standard_normal((count, w.d)) / np.sqrt(w.d)
    else:
        raise ValueError(w.points)
    return p


def _weights(w: Workload, stream: int, count: int) -> np.ndarray:
    if w.weights == "uniform":
        return np.full(count, np.float32(1.0 / count), dtype=np.float32)
    if w.weights == "dirichlet1":
        e = _rng(w.cid, stream).exponential(1.0, size=count)
        return (e / e.sum()).astype(np.float32)
    raise ValueError(w.weights)


@dataclass
class Inputs:
    """Arrays for one workload. x, y are float32, or uint16 bf16 bits when w.dtype == 'bf16'."""
    w: Workload
    x: np.ndarray
    y: np.ndarray
    a: np.ndarray
    b: np.ndarray
    V: Optional[np.ndarray] = None   # m x k, float32
    U: Optional[np.ndarray] = None   # n x k, float32
    extra: dict = field(default_factory=dict)

    def x64(self) -> np.ndarray:
        """x as float64, exactly the stored values."""
        return _stored_to_f64(self.x, self.w.dtype)

    def y64(self) -> np.ndarray:
        return _stored_to_f64(self.y, self.w.dtype)


def _stored_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def _store(p: np.ndarray, dtype: str) -> np.ndarray:
    p32 = np.ascontiguousarray(p, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(p32)
    return p32


def make_inputs(w: Workload, k: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (any n, m: see Workload.scaled)."""
    x = _store(_points(w, STREAM_X, w.n), w.dtype)
    y = _store(_points(w, STREAM_Y, w.m), w.dtype)
    a = _weights(w, STREAM_A, w.n)
    b = _weights(w, STREAM_B, w.m)
    kk = w.apply_k if k is None else k
    V = U = None
    if kk:
        V = _rng(w.cid, STREAM_V).standard_normal((w.m, kk)).astype(np.float32)
        U = _rng(w.cid, STREAM_U).standard_normal((w.n, kk)).astype(np.float32)
    return Inputs(w, x, y, a, b, V, U)


def random_potentials(n: int, m: int, scale: float, seed: int) -> tuple:
    """Seeded float32 potentials, for tests that feed both sides the same (f, g)."""
    rng = np.random.default_rng([seed, 99])
    f = (scale * rng.standard_normal(n)).astype(np.float32)
    g = (scale * rng.standard_normal(m)).astype(np.float32)
    return f, g
