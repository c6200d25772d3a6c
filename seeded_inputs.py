"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module holds no arithmetic of the attention method: it only draws random
numbers, rounds them to the storage dtype and widens stored values back to
float64.  Both sides of every parity check consume the very same host buffers
produced here, so the choice of generator can never affect parity.

Workloads (all synthetic; the pages measure on no public suite):

  c1  B=1,  H=1,  N=M=256,   d=64,  fp32, U[0,1),            non-causal
  c2  B=4,  H=8,  N=M=1024,  d=64,  bf16, N(0,1),            non-causal
  c3  B=2,  H=16, N=M=4096,  d=128, bf16, N(0,1),            causal
  c4  B=1,  H=8,  N=M=16384, d=128, bf16, Q,K N(0,sd=3), V N(0,1), causal
  c5  B=32, H=32, N=1, M=8192, d=128, bf16, N(0,1),          non-causal (decode)

Generator: numpy PCG64 via ``default_rng(seed)``; float32 draws in the order
q, k, v; bf16 storage is round-to-nearest-even of those float32 draws.
The scale is the float32 value of 1/sqrt(d).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    M: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    dist: str           # "uniform01", "normal", "normal_qk3"

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """4*N*M*d per head, halved for causal (the stated metric's convention)."""
        f = 4.0 * self.B * self.H * self.N * self.M * self.d
        return f * 0.5 if self.causal else f

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 256, 64, "f32", False, "uniform01"),
    "c2": Workload("c2", 4, 8, 1024, 1024, 64, "bf16", False, "normal"),
    "c3": Workload("c3", 2, 16, 4096, 4096, 128, "bf16", True, "normal"),
    "c4": Workload("c4", 1, 8, 16384, 16384, 128, "bf16", True, "normal_qk3"),
    "c5": Workload("c5", 32, 32, 1, 8192, 128, "bf16", False, "normal"),
}

# The one-row softmax check that accompanies c1 (logits of the pages' first
# worked example).
C1_SOFTMAX_ROW = np.array([[2.0, 1.0, 0.1]], dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs here are always finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _draw(rng: np.random.Generator, shape, dist: str, which: str) -> np.ndarray:
    if dist == "uniform01":
        return rng.random(shape, dtype=np.float32)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "normal_qk3":
        x = rng.standard_normal(shape, dtype=np.float32)
        return x * np.float32(3.0) if which in ("q", "k") else x
    raise ValueError(f"unknown distribution {dist!r}")


def make_qkv(w: Workload, seed: int):
    """Return (q, k, v) as stored host arrays.

    bf16 workloads give uint16 bit arrays, fp32 workloads float32 arrays.
    Shapes: q [B,H,N,d], k and v [B,H,M,d], C-contiguous.
    """
    rng = np.random.default_rng(seed)
    out = []
    for which, rows in (("q", w.N), ("k", w.M), ("v", w.M)):
        x = _draw(rng, (w.B, w.H, rows, w.d), w.dist, which)
        out.append(f32_to_bf16_bits(x) if w.dtype == "bf16" else x)
    return tuple(out)


def make_rows(rows: int, n: int, seed: int, dist: str = "normal", spread: float = 1.0) -> np.ndarray:
    """float32 [rows, n] logits for the row-wise softmax."""
    rng = np.random.default_rng(seed)
    if dist == "uniform01":
        x = rng.random((rows, n), dtype=np.float32)
    else:
        x = rng.standard_normal((rows, n), dtype=np.float32)
    return (x * np.float32(spread)).astype(np.float32)


def make_bias(shape, seed: int, kind: str = "normal", neg_inf_frac: float = 0.0) -> np.ndarray:
    """float32 additive score bias of `shape` (broadcastable to [B,H,N,M]).

    "normal": N(0, 2^2) entries.  "distance": -slope_h * |i - j| with slopes
    2^(-8 (h+1) / H) over the head axis (a position-distance penalty; the
    shape must be [1,H,N,M]).  neg_inf_frac: that fraction of entries, drawn
    at random, set to -inf (masked keys).
    """
    rng = np.random.default_rng(seed)
    if kind == "normal":
        b = rng.standard_normal(shape, dtype=np.float32) * np.float32(2.0)
    elif kind == "distance":
        _, H, N, M = shape
        slope = np.exp2(-8.0 * (np.arange(H) + 1) / H).reshape(1, H, 1, 1)
        dist = np.abs(np.arange(N).reshape(1, 1, N, 1) - np.arange(M).reshape(1, 1, 1, M))
        b = (-slope * dist).astype(np.float32)
    else:
        raise ValueError(f"unknown bias kind {kind!r}")
    if neg_inf_frac > 0:
        b = np.where(rng.random(b.shape) < neg_inf_frac, np.float32(-np.inf), b).astype(np.float32)
    return np.ascontiguousarray(b)


def sample_rows(w: Workload, count: int, seed: int = 1234) -> np.ndarray:
    """Flat row indices r = (b*H + h)*N + i to sample at full size.

    Always includes the first and last query row of the first and last head
    (the causal extremes), the rest drawn uniformly without replacement.
    """
    total = w.B * w.H * w.N
    rng = np.random.default_rng(seed)
    fixed = {0, w.N - 1, total - w.N, total - 1}
    count = min(count, total)
    extra = rng.choice(total, size=min(total, count + len(fixed)), replace=False)
    rows = sorted(set(int(r) for r in extra[: max(0, count - len(fixed))]) | fixed)
    return np.array(rows[:max(count, len(fixed))], dtype=np.int64)
