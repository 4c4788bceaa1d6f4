"""A GPT-style causal self-attention layer on synthetic data, for timing the autograd path end
to end (the pages quote GPT-style training throughput: page "FlashAttention-2 paper", section
"Three changes").

    y = (attention(x W_qkv split into heads, causal) merged back) W_o

x [B, N, C], W_qkv [C, 3C], W_o [C, C], C = H * d, all bf16 on the GPU. The projections are
torch matmuls (hipBLASLt); the attention is `flash_attn_func` (libfa2.so). Weights and inputs
are random: no data and no trained weights are involved.
"""
from __future__ import annotations

import math

import torch

from .autograd import flash_attn_func


def make_params(B: int, N: int, H: int, d: int, device, seed: int = 0):
    """Random bf16 input, weights (scaled 1/sqrt(C)) and output cotangent, leaf tensors that
    require grad."""
    C = H * d
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda *shape, s=1.0: (torch.randn(*shape, generator=g) * s).to(torch.bfloat16).to(device)
    x = mk(B, N, C).requires_grad_()
    w_qkv = mk(C, 3 * C, s=1.0 / math.sqrt(C)).requires_grad_()
    w_o = mk(C, C, s=1.0 / math.sqrt(C)).requires_grad_()
    dy = mk(B, N, C)
    return x, w_qkv, w_o, dy


def layer_forward(x, w_qkv, w_o, H: int, attn=flash_attn_func, keep=None):
    """Forward of the layer. `attn(q, k, v, causal=True)` takes [B, H, N, d] tensors; `keep`, if
    a dict, receives q, k, v and o (for tests)."""
    B, N, C = x.shape
    d = C // H
    qkv = (x @ w_qkv).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4)  # [3, B, H, N, d]
    q, k, v = (t.contiguous() for t in qkv)
    o = attn(q, k, v, causal=True)
    if keep is not None:
        keep.update(q=q, k=k, v=v, o=o)
    return o.permute(0, 2, 1, 3).reshape(B, N, C) @ w_o


def layer_flop(B: int, N: int, H: int, d: int) -> dict:
    """Nominal FLOP of one forward+backward step: projections (2 matmul FLOP per MAC, backward
    twice the forward) and causal attention (forward 2*B*H*N^2*d, backward 2.5x)."""
    C = H * d
    proj_fwd = 2.0 * B * N * C * 3 * C + 2.0 * B * N * C * C
    attn_fwd = 4.0 * B * H * N * N * d / 2
    return {"projections": 3.0 * proj_fwd, "attention": 3.5 * attn_fwd}
