"""Float64 model of the tiled online-softmax recurrence (no GPU code, no blocking beyond the
tiles the recurrence itself names).

TEST INFRASTRUCTURE: the tests check that this streaming recurrence is the same function as
the plain definition in `oracle.attention`, for several tile shapes, both visiting orders
and with the rescale deferred.

It follows the forward recurrence on page "Flash Attention v2", section "Detailed Algorithm
Comparison / Forward Pass Comparison" (and the seven-step tiled algorithm on page
"flashattention-2", "How FlashAttention-2 Works"): for a block of query rows keep a running
row maximum m, a running sum l and an unnormalised accumulator acc; for each key/value
block compute the block scores, raise m to the new row maximum, rescale l and acc by
exp(m_old - m_new), add exp(scores - m_new) to l and exp(scores - m_new) V to acc. After the
last block O = acc / l and LSE = m + log l. Readings taken where the pages are loose:

* The v2 listing on that page never divides by l; without the division the result is not a
  softmax, so the division is applied once at the end (the deferred normalisation).
* "Delays and batches the rescaling" (page "FlashAttention-2 paper", "Three changes"): with
  `rescale_threshold` = t > 0 the running maximum is only raised when a block's maximum
  exceeds it by more than t (natural-log units), so most blocks skip the rescale; the
  exponentials then stay below exp(t). The result is the same function.
* A row that has not yet seen any visible key (possible when blocks are visited in reverse
  under the causal mask) contributes nothing and keeps m = -inf; the -inf - (-inf) case is
  never evaluated.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["online_attention_forward"]


def online_attention_forward(q, k, v, causal=False, scale=None, block_rows=64, block_cols=64,
                             reverse=False, rescale_threshold=0.0):
    """Tiled forward for q, k, v of shape [N, d] (one batch/head). Returns (O, LSE)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.empty((n, d))
    lse = np.empty(n)
    col_starts = list(range(0, n, block_cols))
    if reverse:
        col_starts = col_starts[::-1]
    for r0 in range(0, n, block_rows):
        rows = np.arange(r0, min(n, r0 + block_rows))
        qi = q[rows]
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), d))
        for c0 in col_starts:
            cols = np.arange(c0, min(n, c0 + block_cols))
            s = scale * (qi @ k[cols].T)
            if causal:
                s[cols[None, :] > rows[:, None]] = -np.inf
            block_max = s.max(axis=1)
            raise_max = block_max > m + rescale_threshold
            m_new = np.where(raise_max, np.maximum(m, block_max), m)
            seen = np.isfinite(m_new)
            alpha = np.ones(len(rows))
            alpha[seen] = np.exp(m[seen] - m_new[seen])  # exp(-inf) = 0 on first sight
            p = np.zeros_like(s)
            p[seen] = np.exp(s[seen] - m_new[seen, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse
