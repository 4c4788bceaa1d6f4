"""torch.autograd face of the fa2 C ABI.

`flash_attn_func(q, k, v, causal, scale)` mirrors the pages' call of the same name (page
"Flash Attention v2", "Installation and Usage": the output of exact attention, with the
backward wired to the FlashAttention-2 backward kernels). Layout here is the library's: bf16 [B, H, N, d],
contiguous, on the GPU. Forward saves q, k, v, O and the per-row LSE; backward calls fa2_bwd
with the incoming dO. Both run through libfa2.so (there is no fallback).
"""
from __future__ import annotations

import torch

from . import ops


class FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float | None, dropout_p: float, seed: int,
                offset: int):
        o, lse = ops.fwd(q, k, v, causal=causal, scale=scale, dropout_p=dropout_p, seed=seed,
                         offset=offset)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, scale, dropout_p, seed, offset)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        causal, scale, p, seed, offset = ctx.args
        dq, dk, dv = ops.bwd(q, k, v, o, do.contiguous(), lse, causal=causal, scale=scale,
                             dropout_p=p, seed=seed, offset=offset)
        return dq, dk, dv, None, None, None, None, None


def flash_attn_func(q, k, v, dropout_p: float = 0.0, causal: bool = False,
                    scale: float | None = None, seed: int = 0, offset: int = 0):
    """softmax(scale * q k^T [+ causal mask]) v for bf16 [B, H, N, d] tensors, differentiable
    in q, k and v. `scale` defaults to 1/sqrt(d). k and v may have Hkv heads with Hkv dividing
    H (query head h uses K/V head h / (H / Hkv)). dropout_p > 0 drops attention probabilities
    with the counter-based mask of (seed, offset); pass a new offset for every call that
    should draw a fresh mask."""
    return FlashAttention.apply(q, k, v, bool(causal), scale, float(dropout_p), int(seed),
                                int(offset))


class FlashAttentionKVPacked(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, kv, causal: bool, scale: float | None):
        o, lse = ops.fwd_kvpacked(q, kv, causal=causal, scale=scale)
        ctx.save_for_backward(q, kv, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, kv, o, lse = ctx.saved_tensors
        dq, dkv = ops.bwd_kvpacked(q, kv, o, do.contiguous(), lse, causal=ctx.causal,
                                   scale=ctx.scale)
        return dq, dkv, None, None


def flash_attn_kvpacked_func(q, kv, causal: bool = False, scale: float | None = None):
    """As flash_attn_func with K and V packed in one bf16 [B, 2, Hkv, N, d] tensor."""
    return FlashAttentionKVPacked.apply(q, kv, bool(causal), scale)
