"""Attention with dropout on the probabilities, in float64, and its mask generator.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module; the HIP library and its binding never do.

What it follows
---------------
The pages' call takes a dropout probability (page "Flash Attention v2", "Installation and
Usage": flash_attn_func(q, k, v, dropout_p=..., ...)) without defining it further. Reading
(the usual one for attention dropout): each probability P[i, j] is kept with probability
1 - p and scaled by 1 / (1 - p), or zeroed, before it multiplies V; the softmax itself and
the saved LSE are those of the undropped scores.

    Z[i, j] in {0, 1} from the counter-based generator below, keep scale s = 1 / P(keep)
    O = (P * Z * s) V,   LSE as without dropout
    backward: dV = (P * Z * s)^T dO,  dP = Z * s * (dO V^T),  D_i = sum_c dO[i, c] O[i, c],
              dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q

The generator is a counter-based one so that the mask can be recomputed anywhere from
(seed, offset, head, i, j) without storing it. It is built from one published 32-bit hash,
the PCG-based hash of Jarzynski and Olano ("Hash Functions for GPU Rendering", Journal of
Computer Graphics Techniques 9(3), 2020):

    h(x):  state = x * 747796405 + 2891336453
           word  = ((state >> ((state >> 28) + 4)) ^ state) * 277803737
           return (word >> 22) ^ word                          (all uint32, wrapping)

    head key   a = h(s0 ^ h(o0 ^ bh)),  s0 = h(seed_lo ^ h(seed_hi)), o0 = h(off_lo ^ h(off_hi))
               (bh = b * H + h, the query head)
    row key    r_i = h(a ^ i)
    pair word  w_im = h(r_i ^ (m * 0x9E3779B9 mod 2^32))   for the key pair m = floor(j / 2)
    uniform    u_ij = low 16 bits of w_im for even j, high 16 bits for odd j
    keep       Z[i, j] = u_ij >= t,  t = floor(p * 2^16),  P(keep) = 1 - t / 2^16

One hash word serves two neighbouring keys (16 bits each), which halves the hashing; the keep
probability is p rounded down to a multiple of 2^-16, and the 1/P(keep) scale uses that
probability, so every output stays unbiased.

Pinned by tests: p = 0 reduces to plain attention exactly; scalar-loop brute force; finite
differences with the mask held fixed; keep rates and independence statistics of the mask;
and that averaging O over many seeds approaches the undropped O (the 1/P(keep) scale).
That h is bit for bit the published function is not pinned (no output values of it are at
hand to compare against); the tests fix its statistics here and, on the GPU, that the kernels'
mask equals this one bit for bit.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, _masked_scores, _row_softmax, resolve_scale

__all__ = ["pcg_hash", "dropout_threshold", "keep_scale", "keep_mask",
           "attention_forward_dropout", "attention_backward_dropout",
           "attention_backward_dropout_sampled"]

_M32 = np.uint64(0xFFFFFFFF)


def pcg_hash(x) -> np.ndarray:
    """The 32-bit hash above, elementwise on uint32 arrays (computed in uint64, masked)."""
    x = np.asarray(x, dtype=np.uint64) & _M32
    state = (x * np.uint64(747796405) + np.uint64(2891336453)) & _M32
    shift = (state >> np.uint64(28)) + np.uint64(4)
    word = (((state >> shift) ^ state) * np.uint64(277803737)) & _M32
    return ((word >> np.uint64(22)) ^ word).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """t = floor(p * 2^16) for 0 <= p < 1."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(p * 65536.0)), 0xFFFF)


def keep_scale(p: float) -> float:
    """1 / P(keep) = 1 / (1 - t / 2^16)."""
    return 1.0 / (1.0 - dropout_threshold(p) / 65536.0)


def _split(x: int):
    x = int(x) & 0xFFFFFFFFFFFFFFFF
    return x & 0xFFFFFFFF, x >> 32


def head_key(seed: int, offset: int, bh: int) -> int:
    s_lo, s_hi = _split(seed)
    o_lo, o_hi = _split(offset)
    s0 = int(pcg_hash(s_lo ^ int(pcg_hash(s_hi))))
    o0 = int(pcg_hash(o_lo ^ int(pcg_hash(o_hi))))
    return int(pcg_hash(s0 ^ int(pcg_hash(o0 ^ (int(bh) & 0xFFFFFFFF)))))


def keep_mask(seed: int, offset: int, bh: int, rows, n_keys: int, p: float) -> np.ndarray:
    """Z[i, j] for the query rows `rows` and keys 0 .. n_keys-1 of query head bh (bool)."""
    a = np.uint64(head_key(seed, offset, bh))
    rows = np.asarray(rows, dtype=np.uint64)
    r = pcg_hash(a ^ rows).astype(np.uint64)                              # [R]
    j = np.arange(n_keys, dtype=np.uint64)
    mm = ((j >> np.uint64(1)) * np.uint64(0x9E3779B9)) & _M32             # pair term [N]
    w = pcg_hash(r[:, None] ^ mm[None, :])                                # [R, N]
    u = np.where((j & np.uint64(1)) == 0, w & np.uint32(0xFFFF), w >> np.uint32(16))
    return u >= np.uint32(dropout_threshold(p))


def _head_ids(B: int, H: int, bh_index):
    """The mask's query-head index of slice (b, h): b*H + h unless given ([B, H] integers,
    for slices cut out of a larger batch)."""
    if bh_index is None:
        return np.arange(B * H).reshape(B, H)
    ids = np.asarray(bh_index, dtype=np.int64)
    if ids.shape != (B, H):
        raise ValueError("bh_index must have shape [B, H]")
    return ids


def attention_forward_dropout(q, k, v, causal: bool = False, scale=None, p: float = 0.0,
                              seed: int = 0, offset: int = 0, rows=None, row_chunk: int = 512,
                              bh_index=None):
    """(O, LSE) of attention with dropout on P; q, k, v [B, H, N, d]. LSE is the undropped
    softmax's. rows: optional subset of query rows. bh_index: see _head_ids."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    s_keep = keep_scale(p)
    row_ids = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_ids.shape[0]
    ids = _head_ids(B, H, bh_index)
    o = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            for c0 in range(0, R, row_chunk):
                ri = row_ids[c0:c0 + row_chunk]
                pr, l = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                z = keep_mask(seed, offset, ids[b, h], ri, N, p)
                o[b, h, c0:c0 + len(ri)] = (pr * z * s_keep) @ v[b, h]
                lse[b, h, c0:c0 + len(ri)] = l
    return o, lse


def attention_backward_dropout(q, k, v, dout, causal: bool = False, scale=None, p: float = 0.0,
                               seed: int = 0, offset: int = 0, row_chunk: int = 512,
                               bh_index=None, o=None):
    """(dQ, dK, dV) of attention_forward_dropout against the cotangent dO. o: optional
    [B, H, N, d], the output handed to a backward pass that takes O as an input; D_i is then
    formed from it (None: the exact dropped O, giving the exact gradient)."""
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    o_in = None if o is None else _as64(o)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    s_keep = keep_scale(p)
    ids = _head_ids(B, H, bh_index)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for c0 in range(0, N, row_chunk):
                ri = np.arange(c0, min(N, c0 + row_chunk))
                pr, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                zs = keep_mask(seed, offset, ids[b, h], ri, N, p) * s_keep
                pd = pr * zs
                o_rows = pd @ v[b, h]
                do_rows = dout[b, h, ri]
                dv[b, h] += pd.T @ do_rows
                dp = zs * (do_rows @ v[b, h].T)
                if o_in is not None:
                    o_rows = o_in[b, h, ri]
                dvec = np.sum(do_rows * o_rows, axis=1, keepdims=True)
                ds = pr * (dp - dvec)
                dq[b, h, ri] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, ri])
    return dq, dk, dv


def attention_backward_dropout_sampled(q, k, v, dout, rows, keys, causal: bool = False,
                                       scale=None, p: float = 0.0, seed: int = 0, offset: int = 0,
                                       row_chunk: int = 256, bh_index=None):
    """attention_backward_dropout restricted to some outputs, for problems too large for the
    whole backward: dQ at the query rows `rows`, dK and dV at the key rows `keys`.

    As the whole backward, row by row: each visited row's softmax and mask are taken over all
    its keys. dQ_i needs row i alone; dK_j and dV_j sum over the query rows that see key j, and
    under the causal mask rows i < j contribute exactly zero, so only rows from min(keys) on are
    visited. Returns float64 [B, H, len(rows), d], [B, H, len(keys), d], [B, H, len(keys), d].
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, N, d = q.shape
    scale = resolve_scale(d, scale)
    s_keep = keep_scale(p)
    ids = _head_ids(B, H, bh_index)
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
                pr, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                zs = keep_mask(seed, offset, ids[b, h], ri, N, p) * s_keep
                do_rows = dout[b, h, ri]
                dvec = np.sum(do_rows * ((pr * zs) @ v[b, h]), axis=1, keepdims=True)
                ds = pr * (zs * (do_rows @ v[b, h].T) - dvec)
                dq[b, h, c0:c0 + len(ri)] = scale * (ds @ k[b, h])
            if not len(keys):
                continue
            for c0 in range(first, N, row_chunk):
                ri = np.arange(c0, min(N, c0 + row_chunk))
                pr, _ = _row_softmax(_masked_scores(q[b, h, ri], ri, k[b, h], causal, scale))
                zs = keep_mask(seed, offset, ids[b, h], ri, N, p) * s_keep
                do_rows = dout[b, h, ri]
                dvec = np.sum(do_rows * ((pr * zs) @ v[b, h]), axis=1, keepdims=True)
                pk, zk = pr[:, keys], zs[:, keys]
                dsk = pk * (zk * (do_rows @ v[b, h, keys].T) - dvec)
                dv[b, h] += (pk * zk).T @ do_rows
                dk[b, h] += scale * (dsk.T @ q[b, h, ri])
    return dq, dk, dv

