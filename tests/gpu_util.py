"""Helpers for the GPU parity tests: move seeded bf16 bits to the device, run the HIP path
through the binding, and compare against the CPU float64 oracle with the stated bounds.

Bounds (bf16 outputs, N(0,1) inputs): max|dO| <= 1e-2, mean|dO| <= 1e-3 over the compared
elements, max|dLSE| <= 1e-3; for each gradient max|g - g_ref| <= 2e-2 * max|g_ref|.
"""
from __future__ import annotations

import numpy as np
import torch

from exact_io_aware_42_amd.inputs import bf16_bits_to_f64

O_MAX = 1e-2
O_MEAN = 1e-3
LSE_MAX = 1e-3
GRAD_REL = 2e-2


def dev():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().double().numpy()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_fwd_close(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray,
                     lse_ref: np.ndarray, what: str = ""):
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), f"{what}: non-finite output"
    e = np.abs(o_gpu - o_ref)
    el = np.abs(lse_gpu - lse_ref)
    info = (f"{what}: max|dO|={e.max():.3e} mean|dO|={e.mean():.3e} max|dLSE|={el.max():.3e} "
            f"worst at {np.unravel_index(e.argmax(), e.shape)}")
    print(info, flush=True)
    assert e.max() <= O_MAX, info
    assert e.mean() <= O_MEAN, info
    assert el.max() <= LSE_MAX, info


def assert_fwd_within_rounding_bound(o_gpu, lse_gpu, o_ref, o_abs_ref, lse_ref, what=""):
    """Bound for inputs outside N(0, 1) (stress cases) and for dropout (kept weights scaled by
    1/P(keep)), derived from the arithmetic: with bf16
    p (unit roundoff u = 2^-8) normalised by the sum of the same rounded p, the weights are
    w_k (1 + e_k) / (1 + sum_j w_j e_j) with |e_k| <= u, so |O' - O| <= 2u sum_k w_k |v_k| (to
    first order); the bf16 output adds at most u |O|. sum_k w_k |v_k| is the oracle's output
    for |V| (o_abs_ref; with dropout the w_k include the mask and the keep scale). LSE keeps
    its 1e-3 bound."""
    u = 2.0 ** -8
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), f"{what}: non-finite output"
    bound = 2 * u * o_abs_ref * 1.01 + u * np.abs(o_ref) + 1e-6
    e = np.abs(o_gpu - o_ref)
    ratio = (e / bound).max()
    el = np.abs(lse_gpu - lse_ref).max()
    info = f"{what}: max|dO|={e.max():.3e} max(|dO|/bound)={ratio:.3f} max|dLSE|={el:.3e}"
    print(info, flush=True)
    assert ratio <= 1.0, info
    assert el <= LSE_MAX, info


def assert_grad_close(got: np.ndarray, want: np.ndarray, what: str):
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    rel = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
    print(f"{what}: max|dg|/max|g| = {rel:.3e}", flush=True)
    assert rel <= GRAD_REL, f"{what}: relative error {rel:.3e} > {GRAD_REL}"


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Query rows to check at full size: the first rows (few visible keys under the causal
    mask), tile boundaries, the last rows, and a seeded random set."""
    fixed = [0, 1, 2, 3, 31, 32, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.choice(N, size=min(count, N), replace=False)
    rows = np.unique(np.concatenate([np.array([r for r in fixed if 0 <= r < N]), rnd]))
    return rows
