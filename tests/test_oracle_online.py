"""The tiled online-softmax recurrence (float64 model) is the same function as the plain
definition, for several tile shapes, both visiting orders, ragged tails and a deferred
rescale; and the shared input generator rounds like PyTorch's bfloat16 conversion."""
import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import (bf16_bits_to_f64, f32_to_bf16_bits, normal_bf16)
from oracle import attention_forward, online_attention_forward


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 8), (16, 16), (32, 8), (64, 128)])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("tau", [0.0, 5.545])
def test_online_equals_definition(causal, br, bc, reverse, tau):
    rng = np.random.default_rng(300 + br + bc)
    n, d = 77, 16  # 77: ragged for every tile size above
    q, k, v = (rng.standard_normal((n, d)) * s for s in (3.0, 3.0, 1.0))
    o_ref, lse_ref = attention_forward(q[None, None], k[None, None], v[None, None], causal=causal)
    o, lse = online_attention_forward(q, k, v, causal=causal, block_rows=br, block_cols=bc,
                                      reverse=reverse, rescale_threshold=tau)
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[0, 0], rtol=0, atol=1e-12)


def test_deferred_rescale_skips_most_rescales():
    """With threshold t the exponentials stay below exp(t); the running max is stale but
    the result is unchanged (checked above). Here: the bound on the exponentials holds."""
    rng = np.random.default_rng(310)
    q, k = rng.standard_normal((64, 8)), rng.standard_normal((64, 8))
    s = q @ k.T / np.sqrt(8)
    tau = 5.545
    m = np.full(64, -np.inf)
    for c0 in range(0, 64, 16):
        bm = s[:, c0:c0 + 16].max(1)
        m = np.where(bm > m + tau, np.maximum(m, bm), m)
        assert (np.exp(s[:, c0:c0 + 16] - m[:, None]) <= np.exp(tau) + 1e-12).all()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(320)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0,
                                  -0.0, 65504.0, 1e-40], dtype=np.float32)])
    ours = f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    back = bf16_bits_to_f64(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_generator_is_seeded_and_normal():
    a = normal_bf16((4, 1000), 7)
    b = normal_bf16((4, 1000), 7)
    c = normal_bf16((4, 1000), 8)
    np.testing.assert_array_equal(a, b)
    assert (a != c).any()
    x = bf16_bits_to_f64(a)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
