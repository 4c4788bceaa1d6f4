"""Pins for the CPU oracle's forward pass: brute force, hand-worked values, closed forms,
invariants and an independent library implementation (PyTorch CPU float64 SDPA).

Each pin is chosen so that a plausible slip in the oracle fails it: a transposed operand
(non-symmetric hand example, SDPA), a wrong mask direction (causal row 0, prefix means),
a missing scale (scale=0 and SDPA with a non-default scale), a dropped max-subtraction
(large-score shift invariance), a wrong LSE (closed forms ln N, ln(i+1)).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_bruteforce, attention_forward, attention_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _parse(x):
    """Golden values are numbers or strings like 'ln3', '-0.75ln3'."""
    if isinstance(x, list):
        return [_parse(y) for y in x]
    if isinstance(x, str):
        coef, _, arg = x.partition("ln")
        c = {"": 1.0, "-": -1.0}.get(coef, None)
        c = float(coef) if c is None else c
        return c * math.log(float(arg))
    return float(x)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ex", range(2))
def test_hand_examples_forward(ex, causal):
    e = _golden()[ex]
    q, k, v = (np.array(_parse(e[t]))[None, None] for t in ("q", "k", "v"))
    ref = e["causal" if causal else "noncausal"]
    o, lse = attention_forward(q, k, v, causal=causal, scale=e["scale"])
    np.testing.assert_allclose(o[0, 0], np.array(_parse(ref["o"])), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.array(_parse(ref["lse"])), rtol=0, atol=1e-14)


@pytest.mark.parametrize("scale", [0.7, -0.7])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 1), (3, 2), (5, 4), (8, 4), (8, 3)])
def test_matches_bruteforce(n, d, causal, scale):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), causal=causal, scale=scale)
    o, lse = attention_forward(q[None, None], k[None, None], v[None, None], causal=causal,
                               scale=scale)
    np.testing.assert_allclose(o[0, 0], np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(lb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [None, 0.3, -0.3])
def test_matches_torch_sdpa(causal, scale):
    """torch's CPU scaled_dot_product_attention (PyTorch's built-in attention, page
    'flashattention-2', 'Adoption') is an implementation written independently of this one."""
    shape = (2, 3, 37, 16)
    q, k, v = _rand(shape, 11), _rand(shape, 12), _rand(shape, 13)
    o, lse = attention_forward(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    # the causal mask as an explicit boolean mask (torch's is_causal path returns NaN for a
    # negative scale: it masks with -inf before the scale multiplies)
    mask = torch.ones(37, 37, dtype=torch.bool).tril() if causal else None
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                          scale=scale)
    np.testing.assert_allclose(o, to.numpy(), rtol=0, atol=1e-12)
    # LSE against torch.logsumexp over the explicitly masked scores
    sc = (1 / math.sqrt(16)) if scale is None else scale
    s = sc * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k = _rand((2, 2, 33, 8), 21, 3.0), _rand((2, 2, 33, 8), 22, 3.0)
    p = attention_probs(q, k, causal=causal)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()
    if causal:
        assert (p[..., np.triu_indices(33, 1)[0], np.triu_indices(33, 1)[1]] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_mean_of_values(causal):
    """Q = 0 makes every visible score 0: uniform weights. Non-causal row i is the mean of
    all V rows and LSE = ln N; causal row i is the prefix mean of V[0..i], LSE = ln(i+1)."""
    n = 19
    q = np.zeros((1, 2, n, 8))
    k, v = _rand((1, 2, n, 8), 31), _rand((1, 2, n, 8), 32)
    o, lse = attention_forward(q, k, v, causal=causal)
    if causal:
        exp_o = np.cumsum(v, axis=2) / np.arange(1, n + 1)[None, None, :, None]
        exp_lse = np.log(np.arange(1, n + 1))[None, None].repeat(2, 1)
    else:
        exp_o = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        exp_lse = np.full((1, 2, n), math.log(n))
    np.testing.assert_allclose(o, exp_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-13)


def test_zero_scale_gives_mean_of_values():
    q, k, v = _rand((1, 1, 7, 4), 41), _rand((1, 1, 7, 4), 42), _rand((1, 1, 7, 4), 43)
    o, lse = attention_forward(q, k, v, scale=0.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (7, 4)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(7), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key_gives_values(causal):
    q, k, v = _rand((2, 3, 1, 5), 51), _rand((2, 3, 1, 5), 52), _rand((2, 3, 1, 5), 53)
    o, lse = attention_forward(q, k, v, causal=causal, scale=0.9)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.9 * np.sum(q * k, -1), rtol=0, atol=1e-14)


def test_causal_row_zero_is_first_value_row():
    q, k, v = _rand((2, 2, 40, 8), 61), _rand((2, 2, 40, 8), 62), _rand((2, 2, 40, 8), 63)
    o, lse = attention_forward(q, k, v, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], np.sum(q[:, :, 0] * k[:, :, 0], -1) / math.sqrt(8),
                               rtol=0, atol=1e-14)
    # and the last causal row equals the non-causal last row
    o_nc, lse_nc = attention_forward(q, k, v, causal=False)
    np.testing.assert_allclose(o[:, :, -1], o_nc[:, :, -1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, -1], lse_nc[:, :, -1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_score_shift_invariance(causal):
    """K' = K + 1 u^T adds scale*(q_i . u) to every score of row i: O unchanged,
    LSE' = LSE + scale * Q u. A large u also checks the max-subtraction (exp would overflow)."""
    q, k, v = _rand((1, 2, 24, 8), 71), _rand((1, 2, 24, 8), 72), _rand((1, 2, 24, 8), 73)
    u = _rand((8,), 74) * 400.0
    o, lse = attention_forward(q, k, v, causal=causal)
    o2, lse2 = attention_forward(q, k + u, v, causal=causal)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse2, lse + (q @ u) / math.sqrt(8), rtol=1e-12, atol=1e-9)


def test_noncausal_permutation_equivariance():
    q, k, v = _rand((1, 1, 16, 4), 81), _rand((1, 1, 16, 4), 82), _rand((1, 1, 16, 4), 83)
    o, lse = attention_forward(q, k, v)
    pk = np.random.default_rng(84).permutation(16)
    pq = np.random.default_rng(85).permutation(16)
    o2, lse2 = attention_forward(q[:, :, pq], k[:, :, pk], v[:, :, pk])
    np.testing.assert_allclose(o2, o[:, :, pq], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, pq], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_convex_hull_and_linearity_in_values(causal):
    q, k = _rand((1, 2, 20, 6), 91, 2.0), _rand((1, 2, 20, 6), 92, 2.0)
    v1, v2 = _rand((1, 2, 20, 6), 93), _rand((1, 2, 20, 6), 94)
    o1, _ = attention_forward(q, k, v1, causal=causal)
    o2, _ = attention_forward(q, k, v2, causal=causal)
    o3, _ = attention_forward(q, k, 2.0 * v1 - 3.0 * v2, causal=causal)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=0, atol=1e-12)
    for i in range(20):
        vis = v1[:, :, : i + 1] if causal else v1
        assert (o1[:, :, i] <= vis.max(axis=2) + 1e-12).all()
        assert (o1[:, :, i] >= vis.min(axis=2) - 1e-12).all()
    # equal value rows: output is that row
    vv = np.broadcast_to(v1[:, :, :1], v1.shape)
    o4, _ = attention_forward(q, k, vv, causal=causal)
    np.testing.assert_allclose(o4, vv, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_chunking_and_row_subsets(causal):
    q, k, v = _rand((1, 2, 70, 8), 101), _rand((1, 2, 70, 8), 102), _rand((1, 2, 70, 8), 103)
    o, lse = attention_forward(q, k, v, causal=causal, row_chunk=1000)
    o2, lse2 = attention_forward(q, k, v, causal=causal, row_chunk=7)
    # BLAS may block differently per chunk size: equal up to rounding
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)
    rows = np.array([69, 0, 33, 5])
    o3, lse3 = attention_forward(q, k, v, causal=causal, rows=rows, row_chunk=3)
    np.testing.assert_allclose(o3, o[:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3, lse[:, :, rows], rtol=0, atol=1e-13)
