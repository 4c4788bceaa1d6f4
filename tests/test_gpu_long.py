"""Sequences beyond 2^16 rows: query and key indices above 65536 in every kernel, on sampled
outputs the CPU oracle computes one by one.

  * N = 100003, d = 128, causal: O and LSE at sampled query rows (first and last rows, the rows
    around 65536, random ones); dQ at the same rows (those with at least 8 visible keys: with
    fewer, the exact dQ can cancel to near zero, which the seeded sweep covers on its own
    terms); dK and dV at sampled keys among the last 1500, which only the query rows from there
    on see, so the oracle visits those rows alone.
  * N = 70001, d = 64, without the mask: O, LSE and dQ at sampled rows (dK and dV at any key
    would need every row's softmax: the whole O(N^2) backward).
  * N = 70001, d = 256, causal: as the first case.
  * N = 70001, d = 128, causal, dropout p = 0.2: O and LSE at sampled rows (held to the rounding
    bound the dropout tests use), dQ at them and dK, dV at sampled keys among the last 1000, whose
    keep bits hash query and key-pair indices past 2^16.

Bounds as everywhere: max|dO| <= 1e-2, mean|dO| <= 1e-3, |dLSE| <= 1e-3 over the sampled rows,
and max|dg| <= 2e-2 * max|g| over the sampled rows or keys.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import bf16_bits_to_f64, default_scale, normal_bf16
from oracle import (attention_backward_dropout_sampled, attention_backward_sampled,
                    attention_forward, attention_forward_dropout)

from gpu_util import (assert_fwd_close, assert_fwd_within_rounding_bound, assert_grad_close,
                      bf16_to_f64, to_dev)

pytestmark = pytest.mark.gpu

CASES = [(1, 1, 100003, 128, True), (1, 2, 70001, 64, False), (1, 1, 70001, 256, True)]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[2]}-d{c[3]}-{'causal' if c[4] else 'full'}"
                                              for c in CASES])
def test_long_sequence_sampled(case):
    import exact_io_aware_42_amd as fa2
    B, H, N, d, causal = case
    seed = 9300 + d
    print(f"case B={B} H={H} N={N} d={d} causal={causal} seed={seed}", flush=True)
    shape = (B, H, N, d)
    bq, bk, bv, bdo = (normal_bf16(shape, seed + t) for t in range(4))
    q, k, v, do = (to_dev(x) for x in (bq, bk, bv, bdo))
    scale = default_scale(d)
    o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    print("fwd and bwd done", flush=True)

    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 2, 7, 8, 65535, 65536, 65537, N - 3, N - 2, N - 1],
                                     rng.integers(0, N, 40)]))
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (bq, bk, bv, bdo))
    o_ref, lse_ref = attention_forward(q64, k64, v64, causal=causal, scale=scale, rows=rows)
    assert_fwd_close(bf16_to_f64(o[:, :, rows]), lse[:, :, rows].cpu().double().numpy(), o_ref,
                     lse_ref, f"N={N} d={d} sampled rows")

    dq_rows = rows[rows >= 8] if causal else rows
    keys = (np.unique(np.concatenate([[N - 1500, N - 2, N - 1], rng.integers(N - 1500, N, 30)]))
            if causal else np.zeros(0, dtype=np.int64))
    gq, gk, gv = attention_backward_sampled(q64, k64, v64, do64, dq_rows, keys, causal=causal,
                                            scale=scale)
    assert_grad_close(bf16_to_f64(dq[:, :, dq_rows]), gq, f"N={N} dq rows")
    if len(keys):
        assert keys.min() > 65536
        assert_grad_close(bf16_to_f64(dk[:, :, keys]), gk, f"N={N} dk keys")
        assert_grad_close(bf16_to_f64(dv[:, :, keys]), gv, f"N={N} dv keys")


def test_long_sequence_dropout():
    import exact_io_aware_42_amd as fa2
    B, H, N, d = 1, 1, 70001, 128
    p, seed, offset = float(np.float32(0.2)), 9400, 7
    print(f"case B={B} H={H} N={N} d={d} causal=True p={p} seed={seed}", flush=True)
    bq, bk, bv, bdo = (normal_bf16((B, H, N, d), seed + t) for t in range(4))
    q, k, v, do = (to_dev(x) for x in (bq, bk, bv, bdo))
    scale = default_scale(d)
    dkw = dict(dropout_p=p, seed=seed, offset=offset)
    o, lse = fa2.fwd(q, k, v, causal=True, scale=scale, **dkw)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=True, scale=scale, **dkw)
    torch.cuda.synchronize()
    print("fwd and bwd done", flush=True)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 8, 65535, 65536, 65537, N - 2, N - 1],
                                     rng.integers(0, N, 40)]))
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (bq, bk, bv, bdo))
    kw = dict(causal=True, scale=scale, p=p, seed=seed, offset=offset)
    o_ref, lse_ref = attention_forward_dropout(q64, k64, v64, rows=rows, **kw)
    o_abs, _ = attention_forward_dropout(q64, k64, np.abs(v64), rows=rows, **kw)
    assert_fwd_within_rounding_bound(bf16_to_f64(o[:, :, rows]),
                                     lse[:, :, rows].cpu().double().numpy(), o_ref, o_abs, lse_ref,
                                     f"N={N} dropout sampled rows")
    dq_rows = rows[rows >= 8]
    keys = np.unique(np.concatenate([[N - 1000, N - 1], rng.integers(N - 1000, N, 30)]))
    gq, gk, gv = attention_backward_dropout_sampled(q64, k64, v64, do64, dq_rows, keys, **kw)
    assert_grad_close(bf16_to_f64(dq[:, :, dq_rows]), gq, f"N={N} dropout dq rows")
    assert_grad_close(bf16_to_f64(dk[:, :, keys]), gk, f"N={N} dropout dk keys")
    assert_grad_close(bf16_to_f64(dv[:, :, keys]), gv, f"N={N} dropout dv keys")
