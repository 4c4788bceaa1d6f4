"""Pins of the dropout oracle (oracle/dropout.py) against things other than itself:
p = 0 is plain attention; scalar loops on tiny inputs; central finite differences with the
mask held fixed; statistics of the counter-based mask (keep rate, row/column/head
independence, hash output uniformity); the 1/P(keep) scale makes the average over seeds
approach the undropped output."""
import math

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_dropout, attention_forward,
                    attention_forward_dropout, keep_mask, keep_scale, pcg_hash)
from oracle.attention import attention_probs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    q, k, v, do = (_rand((2, 2, 37, 8), 10 + t) for t in range(4))
    o0, l0 = attention_forward(q, k, v, causal=causal)
    o1, l1 = attention_forward_dropout(q, k, v, causal=causal, p=0.0, seed=5, offset=9)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    g0 = attention_backward(q, k, v, do, causal=causal)
    g1 = attention_backward_dropout(q, k, v, do, causal=causal, p=0.0, seed=5, offset=9)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_loops(causal):
    """O[i] = sum_j Z[i,j] P[i,j] v_j / P(keep) with P from explicit exp sums."""
    B, H, N, d, p = 1, 2, 7, 3, 0.4
    q, k, v = (_rand((B, H, N, d), 20 + t) for t in range(3))
    scale = 0.7
    o, lse = attention_forward_dropout(q, k, v, causal=causal, scale=scale, p=p, seed=77,
                                       offset=3)
    s_keep = keep_scale(p)
    for h in range(H):
        z = keep_mask(77, 3, h, np.arange(N), N, p)
        for i in range(N):
            js = [j for j in range(N) if not (causal and j > i)]
            e = {j: math.exp(scale * sum(q[0, h, i, c] * k[0, h, j, c] for c in range(d)))
                 for j in js}
            tot = sum(e.values())
            for c in range(d):
                want = sum(e[j] / tot * z[i, j] * s_keep * v[0, h, j, c] for j in js)
                assert abs(o[0, h, i, c] - want) <= 1e-12
            assert abs(lse[0, h, i] - math.log(tot)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_fixed_mask(causal):
    B, H, N, d, p = 1, 1, 5, 3, 0.3
    q, k, v, do = (_rand((B, H, N, d), 30 + t) for t in range(4))
    kw = dict(causal=causal, scale=0.9, p=p, seed=11, offset=1)
    dq, dk, dv = attention_backward_dropout(q, k, v, do, **kw)
    loss = lambda qq, kk, vv: float(np.sum(attention_forward_dropout(qq, kk, vv, **kw)[0] * do))
    eps = 1e-6
    for x, g, idx in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate_and_independence(p):
    rows, n = 256, 4096
    z = keep_mask(2024, 7, 5, np.arange(rows), n, p)
    keep = 1.0 - p
    sd = math.sqrt(keep * (1 - keep) / z.size)
    assert abs(z.mean() - keep) <= 6 * sd
    # per-row and per-column keep rates spread like binomials (no structured rows/columns)
    row_sd = math.sqrt(keep * (1 - keep) / n)
    assert np.abs(z.mean(axis=1) - keep).max() <= 6 * row_sd
    col_sd = math.sqrt(keep * (1 - keep) / rows)
    assert np.abs(z.mean(axis=0) - keep).max() <= 6 * col_sd
    # neighbouring rows, keys, heads, seeds and offsets agree only by chance: p^2 + (1-p)^2
    agree = p * p + keep * keep
    others = [keep_mask(2024, 7, 5, np.arange(1, rows + 1), n, p),   # shifted rows
              keep_mask(2024, 7, 6, np.arange(rows), n, p),          # next head
              keep_mask(2025, 7, 5, np.arange(rows), n, p),          # next seed
              keep_mask(2024, 8, 5, np.arange(rows), n, p)]          # next offset
    zs = z[:, 1:]
    others.append(np.concatenate([zs, z[:, :1]], axis=1))           # shifted keys
    sd_agree = math.sqrt(agree * (1 - agree) / z.size)
    for other in others:
        assert abs((z == other).mean() - agree) <= 6 * sd_agree


def test_hash_output_uniform():
    """h over 2^20 consecutive inputs: the top 8 bits fall in 256 buckets evenly (chi-square
    at about 6 sigma of its 255 degrees of freedom), and so do the low 8 bits."""
    x = pcg_hash(np.arange(1 << 20, dtype=np.uint32))
    for part in (x >> np.uint32(24), x & np.uint32(255)):
        counts = np.bincount(part.astype(np.int64), minlength=256)
        expected = x.size / 256
        chi2 = float(np.sum((counts - expected) ** 2 / expected))
        assert chi2 <= 255 + 6 * math.sqrt(2 * 255)


def test_pair_halves_uniform_and_independent():
    """The two 16-bit halves of one hash word decide two neighbouring keys: over 2^20 words the
    pairs (top 4 bits of the low half, top 4 bits of the high half) fill 256 buckets evenly, so
    the halves are uniform and independent of each other."""
    x = pcg_hash(np.arange(1 << 20, dtype=np.uint32) * np.uint32(7919))
    lo, hi = (x & np.uint32(0xFFFF)) >> np.uint32(12), x >> np.uint32(28)
    counts = np.bincount((lo * 16 + hi).astype(np.int64), minlength=256)
    expected = x.size / 256
    chi2 = float(np.sum((counts - expected) ** 2 / expected))
    assert chi2 <= 255 + 6 * math.sqrt(2 * 255)


@pytest.mark.parametrize("p", [0.1, 0.37, 0.999])
def test_keep_probability_is_p_rounded_to_2_pow_minus_16(p):
    """P(keep) = 1 - floor(p * 2^16) / 2^16 (p rounded down to the 16-bit grid): the empirical
    keep rate of even and of odd keys each lands within 6 standard errors of it, and the keep
    scale is its reciprocal."""
    t = math.floor(p * 65536)
    keep = 1.0 - t / 65536
    assert keep_scale(p) == pytest.approx(1.0 / keep, rel=1e-15)
    z = keep_mask(99, 3, 1, np.arange(512), 2048, p)
    sd = math.sqrt(keep * (1 - keep) / (z.size / 2))
    for part in (z[:, 0::2], z[:, 1::2]):
        assert abs(part.mean() - keep) <= 6 * sd + 1e-12


def test_average_over_seeds_is_unbiased():
    """E[O_dropout] = O: averaging over 400 seeds lands within 5 standard errors."""
    B, H, N, d, p = 1, 1, 6, 4, 0.5
    q, k, v = (_rand((B, H, N, d), 40 + t) for t in range(3))
    o_ref, _ = attention_forward(q, k, v, causal=True)
    outs = np.stack([attention_forward_dropout(q, k, v, causal=True, p=p, seed=s)[0]
                     for s in range(400)])
    mean = outs.mean(axis=0)
    se = outs.std(axis=0) / math.sqrt(outs.shape[0]) + 1e-12
    assert np.all(np.abs(mean - o_ref) <= 5 * se + 1e-9)
    # and the per-entry variance is what Bernoulli weights give: sum_j P^2 v^2 (s - 1)
    probs = attention_probs(q, k, causal=True)[0, 0]
    var = (probs ** 2) @ (v[0, 0] ** 2) * (keep_scale(p) - 1.0)
    np.testing.assert_allclose(outs.var(axis=0)[0, 0], var, rtol=0.25, atol=1e-3)


def test_sampled_heads_match_the_whole_batch():
    """bh_index lets a slice of a batch use its heads' masks: heads cut out of a [2, 3] batch
    give the same outputs and gradients as the whole batch's computation."""
    B, H, N, d, p = 2, 3, 19, 4, 0.35
    q, k, v, do = (_rand((B, H, N, d), 60 + t) for t in range(4))
    kw = dict(causal=True, p=p, seed=4, offset=8)
    o, lse = attention_forward_dropout(q, k, v, **kw)
    g = attention_backward_dropout(q, k, v, do, **kw)
    for b, h in ((0, 2), (1, 1)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        ids = [[b * H + h]]
        o1, l1 = attention_forward_dropout(sl(q), sl(k), sl(v), bh_index=ids, **kw)
        np.testing.assert_array_equal(o1[0, 0], o[b, h])
        np.testing.assert_array_equal(l1[0, 0], lse[b, h])
        g1 = attention_backward_dropout(sl(q), sl(k), sl(v), sl(do), bh_index=ids, **kw)
        for a_, b_ in zip(g1, g):
            np.testing.assert_array_equal(a_[0, 0], b_[b, h])


@pytest.mark.parametrize("causal", [False, True])
def test_given_output_shift_uses_undropped_p(causal):
    # with dropout dS = P * (Z s dP - D) and P the undropped softmax, so a given O' moves dQ
    # and dK exactly as without dropout: by -scale e_i (P K)_i and -scale P^T (e * Q), with
    # e_i = dO_i.(O'_i - O_i) and O the dropped output; dV does not move
    shape = (2, 2, 19, 8)
    q, k, v, do = (_rand(shape, s) for s in (261, 262, 263, 264))
    kw = dict(causal=causal, p=0.3, seed=11, offset=4)
    o, _ = attention_forward_dropout(q, k, v, **kw)
    o2 = o + 0.05 * _rand(shape, 265)
    g0 = attention_backward_dropout(q, k, v, do, **kw)
    g1 = attention_backward_dropout(q, k, v, do, o=o, **kw)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)
    dq, dk, dv = attention_backward_dropout(q, k, v, do, o=o2, **kw)
    scale = 1.0 / math.sqrt(shape[-1])
    e = np.sum(do * (o2 - o), axis=-1, keepdims=True)
    pk, _ = attention_forward(q, k, k, causal=causal)
    p = attention_probs(q, k, causal=causal)
    np.testing.assert_allclose(dq - g0[0], -scale * e * pk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk - g0[1], -scale * np.swapaxes(p, -1, -2) @ (e * q), rtol=0,
                               atol=1e-12)
    np.testing.assert_allclose(dv, g0[2], rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_is_the_whole_backward_at_those_rows(causal):
    # the sampled form restricts the same definition (mask included): its dQ rows and dK, dV
    # keys must be the whole dropout backward's, which the finite-difference pin fixes
    from oracle import attention_backward_dropout_sampled
    shape = (2, 2, 61, 8)
    q, k, v, do = (_rand(shape, s) for s in (281, 282, 283, 284))
    kw = dict(causal=causal, p=0.3, seed=21, offset=5)
    rows = [0, 2, 17, 60]
    keys = [1, 30, 31, 60]
    dq, dk, dv = attention_backward_dropout(q, k, v, do, **kw)
    sq, sk, sv = attention_backward_dropout_sampled(q, k, v, do, rows, keys, row_chunk=9, **kw)
    np.testing.assert_allclose(sq, dq[:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sk, dk[:, :, keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sv, dv[:, :, keys], rtol=0, atol=1e-13)
