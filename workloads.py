"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only lists the
workload shapes and draws random numbers.  Both the HIP path and the fp64
oracle receive the exact same values from here.

Recipe (stated once, used everywhere):
  * generator ``numpy.random.Generator(PCG64(seed))`` with seed = workload id;
  * draws are float32 ``standard_normal`` in the order Q, K, V, then dOut,
    each of shape [B, H, N, D] (Q, K) or [B, H, N, M] (V, dOut);
  * the 784-token image workload multiplies every draw by 0.5;
  * bf16 workloads round each float32 draw to bf16 with round-to-nearest-even,
    once; the oracle then sees those exact bf16 values widened to float64;
  * the decode workload draws, per step t = 0, 1, ..., the triple
    q_t [B, H, D], k_t [B, H, D], v_t [B, H, M] in that order.

The workloads stand in for the pages' experiments by shape only: 784 and 3072
tokens are the pixel counts of the MNIST and CIFAR-10 image-generation
sequences, 65536 tokens is a long synthetic sequence in the spirit of the
pages' time/memory-vs-length benchmark, and the decode workload is batched
autoregressive generation.  No dataset or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    N: int
    D: int
    M: int
    dtype: str          # "f32" or "bf16": the I/O type of q, k, v, out (and gradients)
    scale: float = 1.0
    steps: int = 0      # decode workloads: number of sequential steps

    def with_n(self, N: int) -> "Workload":
        return replace(self, N=N)

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "small causal+non-causal, B1 H2 N256 D=M=32 f32", 1, 2, 256, 32, 32, "f32"),
    2: Workload(2, "image sequence 784, B16 H8 N784 D=M=32 f32 (x0.5)", 16, 8, 784, 32, 32, "f32", 0.5),
    3: Workload(3, "image sequence 3072, B8 H8 N3072 D=M=32 bf16", 8, 8, 3072, 32, 32, "bf16"),
    4: Workload(4, "long sequence, B1 H8 N65536 D=M=64 bf16, forward+backward", 1, 8, 65536, 64, 64, "bf16"),
    5: Workload(5, "batched decode, B256 H8 D=M=64 bf16 I/O fp32 state, 3072 steps", 256, 8, 1, 64, 64, "bf16",
                steps=3072),
}

# Sequence lengths of the long-sequence sweep (powers of two, 512 .. 65536).
SWEEP_N = [512 * (1 << i) for i in range(8)]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values as the I/O dtype holds them, returned as float32 (exact)."""
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x))
    return np.ascontiguousarray(x, dtype=np.float32)


def forward_inputs(w: Workload, with_dout: bool = False, seed: int | None = None):
    """Q, K, V (and dOut) for a forward/backward workload, as float32 arrays holding
    exactly the I/O-dtype values.  ``seed`` defaults to the workload id."""
    g = rng(w.wid if seed is None else seed)
    shapes = [(w.B, w.H, w.N, w.D), (w.B, w.H, w.N, w.D), (w.B, w.H, w.N, w.M)]
    if with_dout:
        shapes.append((w.B, w.H, w.N, w.M))
    out = []
    for s in shapes:
        x = g.standard_normal(s, dtype=np.float32)
        if w.scale != 1.0:
            x *= np.float32(w.scale)
        out.append(round_to(x, w.dtype))
    return tuple(out)


def start_state(w: Workload, seed: int):
    """An arbitrary fp32 recurrent state to start a causal forward from:
    S0 [B, H, D, M] = 4 x standard normal (any sign), Z0 [B, H, D] =
    5 |standard normal| + 0.5 (positive, so every denominator is positive)."""
    g = rng(seed)
    S0 = g.standard_normal((w.B, w.H, w.D, w.M), dtype=np.float32) * np.float32(4.0)
    Z0 = np.abs(g.standard_normal((w.B, w.H, w.D), dtype=np.float32)) * np.float32(5.0) + np.float32(0.5)
    return np.ascontiguousarray(S0), np.ascontiguousarray(Z0)


def rff_params(D: int, R: int, seed: int, sigma: float | None = None):
    """omega [D, R] ~ N(0, 1/sigma^2) and bias [R] ~ U[0, 2 pi), float32, for
    random Fourier features; sigma defaults to 2 sqrt(D), which keeps the RBF
    kernel of N(0, 1) queries and keys near exp(-1/4) (well-conditioned
    attention)."""
    sigma = 2.0 * np.sqrt(D) if sigma is None else sigma
    g = rng(seed)
    omega = g.standard_normal((D, R), dtype=np.float32) * np.float32(1.0 / sigma)
    bias = g.uniform(0.0, 2.0 * np.pi, R).astype(np.float32)
    return np.ascontiguousarray(omega), np.ascontiguousarray(bias)


class DecodeStream:
    """Per-step decode inputs, drawn in order q_t, k_t, v_t for t = 0, 1, ..."""

    def __init__(self, w: Workload, seed: int | None = None):
        self.w = w
        self.g = rng(w.wid if seed is None else seed)
        self.t = 0

    def next(self):
        w = self.w
        q = self.g.standard_normal((w.B, w.H, w.D), dtype=np.float32)
        k = self.g.standard_normal((w.B, w.H, w.D), dtype=np.float32)
        v = self.g.standard_normal((w.B, w.H, w.M), dtype=np.float32)
        self.t += 1
        return round_to(q, w.dtype), round_to(k, w.dtype), round_to(v, w.dtype)

    def take(self, steps: int):
        """Stack ``steps`` draws: arrays [steps, B, H, D] / [steps, B, H, M] (float32)."""
        w = self.w
        qs = np.empty((steps, w.B, w.H, w.D), np.float32)
        ks = np.empty((steps, w.B, w.H, w.D), np.float32)
        vs = np.empty((steps, w.B, w.H, w.M), np.float32)
        for t in range(steps):
            qs[t], ks[t], vs[t] = self.next()
        return qs, ks, vs
