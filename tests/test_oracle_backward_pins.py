"""Pins for the CPU oracle's analytic backward: hand-worked values, central finite
differences of L = sum(dO * O), PyTorch CPU float64 autograd through SDPA, and gradient
invariants. The finite-difference pin rejects the 'dS = dP * P * (1 - P)' form printed
under "2. Backward Pass Computation" on page "Flash Attention v2" (it is only the diagonal
of the softmax Jacobian); a test below checks that explicitly."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward

from test_oracle_pins import GOLDEN, _parse


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [False, True])
def test_hand_example_backward(causal):
    with open(GOLDEN) as f:
        e = json.load(f)["examples"][0]
    q, k, v, do = (np.array(_parse(e[t]))[None, None] for t in ("q", "k", "v", "dout"))
    ref = e["causal" if causal else "noncausal"]
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=e["scale"])
    for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        np.testing.assert_allclose(got[0, 0], np.array(_parse(ref[key])), rtol=0, atol=1e-14)


def _loss(q, k, v, do, causal, scale):
    o, _ = attention_forward(q, k, v, causal=causal, scale=scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("scale", [0.8, -0.8, 0.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (3, 2), (5, 4), (8, 4)])
def test_finite_differences(n, d, causal, scale):
    shape = (1, 1, n, d)
    q, k, v, do = (_rand(shape, s) for s in (201, 202, 203, 204))
    grads = attention_backward(q, k, v, do, causal=causal, scale=scale)
    h = 1e-6
    for idx, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            num[pos] = (_loss(*args_p, do, causal, scale) - _loss(*args_m, do, causal, scale)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_diagonal_only_softmax_gradient_is_rejected():
    """The 'dS = dP * P * (1 - P)' shortcut differs from the true gradient: the finite
    difference above is what separates them, shown here on one small case."""
    shape = (1, 1, 4, 3)
    q, k, v, do = (_rand(shape, s) for s in (211, 212, 213, 214))
    _, dk_true, _ = attention_backward(q, k, v, do)
    s = q[0, 0] @ k[0, 0].T / math.sqrt(3)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    dk_wrong = (dp * p * (1 - p)).T @ q[0, 0] / math.sqrt(3)
    assert np.max(np.abs(dk_wrong - dk_true[0, 0])) > 1e-3


@pytest.mark.parametrize("scale", [0.2, -0.2])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal, scale):
    shape = (2, 2, 29, 16)
    q, k, v, do = (_rand(shape, s) for s in (221, 222, 223, 224))
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=scale, row_chunk=8)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    # the causal mask as an explicit boolean mask (torch's is_causal path returns NaN for a
    # negative scale: it masks with -inf before the scale multiplies)
    mask = torch.ones(29, 29, dtype=torch.bool).tril() if causal else None
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                          scale=scale)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    shape = (1, 2, 31, 8)
    q, k, v, do = (_rand(shape, s) for s in (231, 232, 233, 234))
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal)
    # rows of dS sum to zero, so the key gradients sum to zero over keys
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # every P row sums to one, so dV summed over keys equals dO summed over queries
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # zero cotangent gives zero gradients
    z = attention_backward(q, k, v, np.zeros_like(do), causal=causal)
    for g in z:
        assert np.max(np.abs(g)) == 0.0
    # identical key rows: scores constant along each row, so dQ = 0
    kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
    dq2, _, _ = attention_backward(q, kk, v, do, causal=causal)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_given_output_one_key_closed_form(causal):
    # one key: P = 1 and the exact O is v, so dS = dO.v - dO.o' = -dO.(o' - v); the gradient
    # at o' = v is zero, and a perturbed o' moves dQ by -scale (dO.delta) k, dK by the same
    # with q, and leaves dV = dO
    shape = (2, 3, 1, 16)
    q, k, v, do = (_rand(shape, s) for s in (241, 242, 243, 244))
    delta = 1e-3 * _rand(shape, 245)
    scale = 0.37
    dq0, dk0, dv0 = attention_backward(q, k, v, do, causal=causal, scale=scale, o=v)
    # (zero up to float64 summation order: dO.v is taken once as a product, once as a sum)
    assert np.abs(dq0).max() <= 1e-14 and np.abs(dk0).max() <= 1e-14
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=scale, o=v + delta)
    proj = np.sum(do * delta, axis=-1, keepdims=True)
    np.testing.assert_allclose(dq, -scale * proj * k, rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dk, -scale * proj * q, rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_given_output_shift_through_forward(causal):
    # D_i moves by e_i = dO_i.(o'_i - O_i); dS_ij moves by -P_ij e_i, so dQ_i moves by
    # -scale e_i sum_j P_ij k_j, which is row i of attention(Q, K, K), and dK_j by
    # -scale sum_i P_ij e_i q_i; dV does not move
    from oracle.attention import attention_probs
    shape = (1, 2, 23, 8)
    q, k, v, do = (_rand(shape, s) for s in (251, 252, 253, 254))
    o, _ = attention_forward(q, k, v, causal=causal)
    o2 = o + 0.05 * _rand(shape, 255)
    g0 = attention_backward(q, k, v, do, causal=causal)
    g1 = attention_backward(q, k, v, do, causal=causal, o=o)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, o=o2)
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
    # the sampled form restricts the same definition: its dQ rows and dK, dV keys must be the
    # whole backward's (which the finite-difference, autograd and hand-worked pins fix),
    # including under the causal mask, where it visits only the rows from the first key on
    from oracle import attention_backward_sampled
    shape = (2, 2, 67, 16)
    q, k, v, do = (_rand(shape, s) for s in (271, 272, 273, 274))
    rows = [0, 1, 5, 33, 66]
    keys = [3, 40, 41, 66]
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal)
    sq, sk, sv = attention_backward_sampled(q, k, v, do, rows, keys, causal=causal, row_chunk=7)
    np.testing.assert_allclose(sq, dq[:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sk, dk[:, :, keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sv, dv[:, :, keys], rtol=0, atol=1e-13)
