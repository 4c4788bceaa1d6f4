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


def assert_grad_close(got: np.ndarray, want: np.ndarray, what: str, bound: float = GRAD_REL,
                      floor: float = 0.0):
    """max|got - want| <= bound * max|want| + floor (floor: an absolute rounding bound for
    gradients whose exact value can cancel to zero)."""
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err, top = np.abs(got - want).max(), np.abs(want).max()
    rel = err / max(top, 1e-30)
    print(f"{what}: max|dg|/max|g| = {rel:.3e} (max|dg| {err:.3e}, floor {floor:.3e})", flush=True)
    assert err <= bound * top + floor, \
        f"{what}: max|dg| {err:.3e} > {bound} * {top:.3e} + {floor:.3e} (relative {rel:.3e})"


def compare_forward_all_heads(bq, bk, bv, o_bits, lse_gpu, causal, scale, what="",
                              workers=None):
    """Every element of O and LSE against the float64 oracle, one (batch, head) slice per
    task on a thread pool (BLAS held to one thread per task, so the pool sets the
    parallelism). o_bits: the GPU's O as bf16 bits [B, H, N, d]; lse_gpu: its LSE [B, H, N].
    The bounds are checked over all elements: max|dO| <= 1e-2, mean|dO| <= 1e-3 and
    max|dLSE| <= 1e-3. Also printed: the worst head, max|dO| over rows >= 16 (rows with many
    visible keys) and the largest |dO| - ulp_bf16(O_ref)/2, the error beyond the output's own
    rounding. Returns the statistics."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention_forward

    B, H, N, d = bq.shape
    G = H // bk.shape[1]
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite LSE"
    workers = workers or min(16, os.cpu_count() or 1)

    def one(bh):
        b, h = divmod(bh, H)
        o_ref, lse_ref = attention_forward(
            bf16_bits_to_f64(bq[b:b + 1, h:h + 1]), bf16_bits_to_f64(bk[b:b + 1, h // G:h // G + 1]),
            bf16_bits_to_f64(bv[b:b + 1, h // G:h // G + 1]), causal=causal, scale=scale)
        o_got = bf16_bits_to_f64(o_bits[b:b + 1, h:h + 1])
        if not np.isfinite(o_got).all():
            return dict(bh=bh, finite=False)
        e = np.abs(o_got - o_ref)[0, 0]
        # half an ulp of bf16 at |O_ref| (8 significant bits): 2^(floor(log2|x|) - 8)
        mag = np.abs(o_ref[0, 0])
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 8)
        return dict(bh=bh, finite=True, max=float(e.max()), sum=float(e.sum()),
                    max16=float(e[16:].max()) if N > 16 else 0.0,
                    beyond=float((e - half_ulp).max()),
                    lse=float(np.abs(lse_gpu[b, h] - lse_ref[0, 0]).max()))

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one, range(B * H)))
    bad = [r["bh"] for r in res if not r["finite"]]
    assert not bad, f"{what}: non-finite O in (batch*head) slices {bad[:8]}"
    worst = max(res, key=lambda r: r["max"])
    st = dict(max=worst["max"], mean=sum(r["sum"] for r in res) / (B * H * N * d),
              lse=max(r["lse"] for r in res), max_rows16=max(r["max16"] for r in res),
              beyond_half_ulp=max(r["beyond"] for r in res), worst_head=worst["bh"],
              elements=B * H * N * d)
    info = (f"{what}: every element ({st['elements']}): max|dO|={st['max']:.3e} "
            f"mean|dO|={st['mean']:.3e} max|dLSE|={st['lse']:.3e}; worst head (b*H+h) "
            f"{st['worst_head']}; rows>=16 max|dO|={st['max_rows16']:.3e}; "
            f"max(|dO| - ulp/2)={st['beyond_half_ulp']:.3e}")
    print(info, flush=True)
    assert st["max"] <= O_MAX, info
    assert st["mean"] <= O_MEAN, info
    assert st["lse"] <= LSE_MAX, info
    return st
