"""Plain CPU float64 attention: the definition written out, forward and analytic backward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module; the HIP library and its binding never do.

What it follows
---------------
Forward (page "Flash Attention v2", section "Flash Attention v1: Recap / What v1 Solved",
the standard-attention listing; page "flashattention-2", "What Is FlashAttention-2?": the
fused method returns exactly this result):

    S = scale * Q K^T                        (scale = 1/sqrt(d) by default; the same page's
                                             "Detailed Algorithm Comparison" divides the
                                             scores by sqrt(d))
    causal: S[i, j] = -inf for j > i        (page "flashattention-2", "FlashAttention-2
                                             Improvements Over v1": the autoregressive mask;
                                             top-left aligned, queries and keys share N)
    P = softmax(S) row by row, O = P V
    LSE[i] = log sum_j exp(S[i, j])         (natural log; the per-row statistic saved for the
                                             backward pass, "Write l_i, m_i to HBM" in the
                                             v1 forward listing, folded into one number)

Backward: the gradient of the forward map above, written from calculus rather than from
any printed listing (the listing under "2. Backward Pass Computation" on page "Flash
Attention v2" keeps only the diagonal of the softmax Jacobian, adds dV twice and drops the
scale; its structure, recompute P block by block and accumulate dQ, dK, dV, is what the
fused kernels follow):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_c dO[i, c] * O[i, c]           (= sum_j P[i, j] dP[i, j])
    dS = P * (dP - D)                        (row-softmax Jacobian applied to dP)
    dQ = scale * dS K,  dK = scale * dS^T Q

A backward pass that takes O as an input (the fused one does; so does this function when
given `o`) forms D from that O. At the exact O it is the gradient above; at an O rounded to
the output format, D and so dS, dQ and dK move by the rounding's dot product with dO, which
in rows of a few keys is not small against the gradient itself.

Precision: float64 throughout; inputs are the exact bf16 values widened to float64.
Query rows are processed in chunks: row i of the result depends only on q_i and the whole
of K and V, so chunking changes nothing but memory use (pinned by a test).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_forward", "attention_backward", "attention_backward_sampled",
           "attention_probs", "resolve_scale"]


def resolve_scale(d: int, scale) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _masked_scores(q_rows: np.ndarray, row_ids: np.ndarray, k: np.ndarray, causal: bool,
                   scale: float) -> np.ndarray:
    """scale * q_rows k^T with keys j > i set to -inf when causal. q_rows [R, d], k [N, d]."""
    s = scale * (q_rows @ k.T)
    if causal:
        n = k.shape[0]
        s[np.arange(n)[None, :] > row_ids[:, None]] = -np.inf
    return s


def _row_softmax(s: np.ndarray):
    """Return (P, LSE) for a block of score rows; every row has at least one finite entry."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_probs(q, k, causal: bool = False, scale=None) -> np.ndarray:
    """P = softmax(scale Q K^T [+ mask]) as a dense [B, H, N, N] array (small sizes only)."""
    q, k = _as64(q), _as64(k)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    rows = np.arange(N)
    p = np.empty((B, H, N, N))
    for b in range(B):
        for h in range(H):
            p[b, h], _ = _row_softmax(_masked_scores(q[b, h], rows, k[b, h], causal, scale))
    return p


def attention_forward(q, k, v, causal: bool = False, scale=None, rows=None,
                      row_chunk: int = 512):
    """Exact attention forward in float64.

    q, k, v: [B, H, N, d] (any real dtype; widened to float64).
    rows: optional 1-D array of query indices; then only those rows are computed and the
    outputs have that many rows (each row is independent of the others).
    Returns (O [B, H, R, d], LSE [B, H, R]) with R = N or len(rows).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    row_ids = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_ids.shape[0]
    o = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            for c0 in range(0, R, row_chunk):
                ri = row_ids[c0:c0 + row_chunk]
                s = _masked_scores(q[b, h, ri], ri, k[b, h], causal, scale)
                p, l = _row_softmax(s)
                o[b, h, c0:c0 + len(ri)] = p @ v[b, h]
                lse[b, h, c0:c0 + len(ri)] = l
    return o, lse


def attention_backward(q, k, v, dout, causal: bool = False, scale=None, row_chunk: int = 512,
                       o=None):
    """Exact gradients (dQ, dK, dV) of O = attention(Q, K, V) against the cotangent dO.

    O and P are recomputed here in float64 from the definition. o: optional [B, H, N, d], the
    output handed to a backward pass that takes O as an input; D_i is then formed from it
    (with o = the exact O this is the exact gradient, as with o = None). Returns three
    float64 arrays of shape [B, H, N, d].
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    o_in = None if o is None else _as64(o)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for c0 in range(0, N, row_chunk):
                ri = np.arange(c0, min(N, c0 + row_chunk))
                p, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                o_rows = p @ v[b, h]
                do_rows = dout[b, h, ri]
                dv[b, h] += p.T @ do_rows
                dp = do_rows @ v[b, h].T
                if o_in is not None:
                    o_rows = o_in[b, h, ri]
                dvec = np.sum(do_rows * o_rows, axis=1, keepdims=True)
                ds = p * (dp - dvec)
                dq[b, h, ri] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, ri])
    return dq, dk, dv


def attention_backward_sampled(q, k, v, dout, rows, keys, causal: bool = False, scale=None,
                               row_chunk: int = 256):
    """attention_backward restricted to some outputs, for problems too large for the whole
    backward: dQ at the query rows `rows`, dK and dV at the key rows `keys`.

    dQ_i depends on row i alone (its softmax over all keys). dK_j and dV_j sum over every query
    row that sees key j; under the causal mask rows i < j have P_ij = 0 exactly, so only rows from
    min(keys) on are visited. Each visited row's softmax is taken over all its keys, as in the
    definition. Returns float64 [B, H, len(rows), d], [B, H, len(keys), d], [B, H, len(keys), d].
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    dq = np.empty((B, H, len(rows), d))
    dk = np.zeros((B, H, len(keys), d))
    dv = np.zeros((B, H, len(keys), d))
    first = int(keys.min()) if causal and len(keys) else 0
    for b in range(B):
        for h in range(H):
            for c0 in range(0, len(rows), row_chunk):
                ri = rows[c0:c0 + row_chunk]
                p, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                do_rows = dout[b, h, ri]
                dvec = np.sum(do_rows * (p @ v[b, h]), axis=1, keepdims=True)
                ds = p * (do_rows @ v[b, h].T - dvec)
                dq[b, h, c0:c0 + len(ri)] = scale * (ds @ k[b, h])
            if not len(keys):
                continue
            for c0 in range(first, N, row_chunk):
                ri = np.arange(c0, min(N, c0 + row_chunk))
                p, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                do_rows = dout[b, h, ri]
                dvec = np.sum(do_rows * (p @ v[b, h]), axis=1, keepdims=True)
                pk = p[:, keys]
                dsk = pk * (do_rows @ v[b, h, keys].T - dvec)
                dv[b, h] += pk.T @ do_rows
                dk[b, h] += scale * (dsk.T @ q[b, h, ri])
    return dq, dk, dv
