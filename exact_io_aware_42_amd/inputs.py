"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the CPU oracle.

This module holds no attention arithmetic. It only draws i.i.d. N(0, 1) float32 values
from a seeded numpy generator, rounds them to bfloat16 with round-to-nearest-even, and
decodes bfloat16 bit patterns back to float64 (a lossless widening). Both sides of a
parity check receive the same bf16 bytes: the GPU as a torch bfloat16 tensor, the
oracle as the exact float64 values of those bytes.

Workload shapes follow the attention workloads measured for FlashAttention-2 (page
"FlashAttention-2 paper", section "Things that break": always name shape, dtype and GPU):
self-attention with Q, K, V of shape [B, H, N, d] in row-major order, d fastest.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f64",
    "bf16_bits_to_f32",
    "normal_bf16",
    "Workload",
    "WORKLOADS",
    "workload_tensors",
    "sha256_hex",
    "default_scale",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Finite inputs only (the generators below never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """bfloat16 bits of sigma * N(0, 1) float32 draws from numpy's PCG64 seeded with `seed`."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f32_to_bf16_bits(x)


def sha256_hex(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d), as the float32 value the kernel receives."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclass(frozen=True)
class Workload:
    """One attention workload: shape, masking modes and the seed base (seed = 1000*id + t,
    t = 1, 2, 3, 4 for Q, K, V, dO)."""

    wid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal_modes: tuple
    backward: bool = False

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def seed(self, t: int) -> int:
        return 1000 * self.wid + t


WORKLOADS = {
    1: Workload(1, "tiny B1 H2 N256 d64", 1, 2, 256, 64, (False, True)),
    2: Workload(2, "B8 H32 N2048 d64", 8, 32, 2048, 64, (False, True)),
    3: Workload(3, "GPT-style B4 H16 N4096 d128", 4, 16, 4096, 128, (True,)),
    4: Workload(4, "long sequence B1 H16 N16384 d128", 1, 16, 16384, 128, (True, False)),
    5: Workload(5, "fwd+bwd B4 H16 N2048 d128", 4, 16, 2048, 128, (True,), backward=True),
    # head dimension 256 (forward), the largest the pages give for FlashAttention-2
    6: Workload(6, "head dim 256 B2 H16 N4096 d256", 2, 16, 4096, 256, (True, False)),
}


def workload_tensors(w: Workload, with_dout: bool = False) -> dict:
    """bf16 bits for q, k, v (and dout) of workload `w`, each [B, H, N, d] uint16."""
    out = {
        "q": normal_bf16(w.shape, w.seed(1)),
        "k": normal_bf16(w.shape, w.seed(2)),
        "v": normal_bf16(w.shape, w.seed(3)),
    }
    if with_dout:
        out["dout"] = normal_bf16(w.shape, w.seed(4))
    return out
