"""Scalar brute-force attention for tiny inputs (pure Python loops, math.exp).

TEST INFRASTRUCTURE: used only by the tests to pin the vectorised oracle on tiny shapes.

Follows the standard-attention definition (page "Flash Attention v2", section "Flash
Attention v1: Recap / What v1 Solved"): every score s_ij = scale * sum_c q_ic k_jc, the
causal mask removes keys j > i, each row is normalised by its own sum of exponentials,
and the output row is the weighted sum of value rows. The row maximum is subtracted before
exponentiating only to keep exp() in range; it cancels in the ratio.
"""
from __future__ import annotations

import math

__all__ = ["attention_bruteforce"]


def attention_bruteforce(q, k, v, causal=False, scale=None):
    """q, k, v: nested lists [N][d] of floats for one (batch, head). Returns (O, LSE) lists."""
    n = len(q)
    d = len(q[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = [], []
    for i in range(n):
        visible = [j for j in range(n) if not (causal and j > i)]
        scores = {j: scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in visible}
        mx = max(scores.values())
        weights = {j: math.exp(s - mx) for j, s in scores.items()}
        total = sum(weights.values())
        out.append([sum(weights[j] * v[j][c] for j in visible) / total for c in range(d)])
        lse.append(mx + math.log(total))
    return out, lse
