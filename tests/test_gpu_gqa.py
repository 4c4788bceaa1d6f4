"""Grouped K/V heads (Hkv dividing H) and packed K/V through the C ABI, against the CPU
float64 oracle: the definition with each K/V head repeated for the query heads of its group;
dK and dV of a K/V head are the sums over its group. Bounds as in the other parity tests."""
import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import bf16_bits_to_f64, default_scale, normal_bf16
from oracle import attention_backward, attention_forward

from gpu_util import assert_fwd_close, assert_grad_close, bf16_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _fa2():
    import exact_io_aware_42_amd as fa2
    return fa2


def _oracle(bq, bk, bv, bdo, causal, scale):
    B, H, N, d = bq.shape
    G = H // bk.shape[1]
    q64, k64, v64, do64 = (bf16_bits_to_f64(b) for b in (bq, bk, bv, bdo))
    kr, vr = np.repeat(k64, G, axis=1), np.repeat(v64, G, axis=1)
    o, lse = attention_forward(q64, kr, vr, causal=causal, scale=scale)
    dq, dk, dv = attention_backward(q64, kr, vr, do64, causal=causal, scale=scale)
    Hkv = H // G
    return o, lse, dq, dk.reshape(B, Hkv, G, N, d).sum(2), dv.reshape(B, Hkv, G, N, d).sum(2)


CASES = [((2, 8, 2, 150, 64), True), ((2, 8, 2, 150, 64), False), ((1, 4, 1, 200, 128), True),
         ((1, 6, 3, 333, 128), False), ((1, 4, 2, 96, 256), True)]


@pytest.mark.parametrize("dims,causal", CASES,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-{'c' if c else 'f'}" for (b, h, hk, n, d), c in CASES])
def test_grouped_heads_match_oracle(dims, causal):
    fa2 = _fa2()
    B, H, Hkv, N, d = dims
    seed = 9300 + H + N + d
    bq, bdo = normal_bf16((B, H, N, d), seed), normal_bf16((B, H, N, d), seed + 3)
    bk, bv = normal_bf16((B, Hkv, N, d), seed + 1), normal_bf16((B, Hkv, N, d), seed + 2)
    scale = default_scale(d)
    print(f"case {dims} causal={causal}", flush=True)
    q, k, v, do = (to_dev(b) for b in (bq, bk, bv, bdo))
    o, lse = fa2.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = _oracle(bq, bk, bv, bdo, causal, scale)
    assert_fwd_close(bf16_to_f64(o), lse.cpu().double().numpy(), o_ref, lse_ref, str(dims))
    for name, got, want in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        assert_grad_close(bf16_to_f64(got), want, f"{dims} {name}")


@pytest.mark.parametrize("causal", [False, True])
def test_packed_and_strided_kv(causal):
    """K/V packed as [B, 2, Hkv, N, d], and K/V taken from a wider buffer (batch stride
    3*Hkv*N*d), give the same bits as separate contiguous tensors; autograd through the packed
    form matches the direct call."""
    fa2 = _fa2()
    B, H, Hkv, N, d = 2, 4, 2, 130, 128
    bq, bdo = normal_bf16((B, H, N, d), 9401), normal_bf16((B, H, N, d), 9404)
    bk, bv = normal_bf16((B, Hkv, N, d), 9402), normal_bf16((B, Hkv, N, d), 9403)
    q, k, v, do = (to_dev(b) for b in (bq, bk, bv, bdo))
    o, lse = fa2.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=causal)
    kv = torch.stack([k, v], dim=1).contiguous()
    o2, lse2 = fa2.fwd_kvpacked(q, kv, causal=causal)
    dq2, dkv2 = fa2.bwd_kvpacked(q, kv, o2, do, lse2, causal=causal)
    wide = torch.zeros((B, 3, Hkv, N, d), dtype=torch.bfloat16, device=q.device)
    wide[:, 0], wide[:, 2] = k, v
    o3, lse3 = fa2.fwd(q, wide[:, 0], wide[:, 2], causal=causal)
    dq3, dk3, dv3 = fa2.bwd(q, wide[:, 0], wide[:, 2], o3, do, lse3, causal=causal)
    qa = q.clone().requires_grad_()
    kva = kv.clone().requires_grad_()
    o4 = fa2.flash_attn_kvpacked_func(qa, kva, causal=causal)
    o4.backward(do)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    for got in (o2, o3, o4.detach()):
        assert same(got, o)
    assert torch.equal(lse2, lse) and torch.equal(lse3, lse)
    for a_, b_ in ((dq2, dq), (dkv2[:, 0], dk), (dkv2[:, 1], dv), (dq3, dq), (dk3, dk), (dv3, dv),
                   (qa.grad, dq), (kva.grad[:, 0], dk), (kva.grad[:, 1], dv)):
        assert same(a_, b_)


def test_grouped_heads_full_size_step():
    """The grouped-head step at the benchmark's shape (B=4, 16 query heads on 4 K/V heads,
    N=2048, d=128, causal), in the benchmark's launch configuration: for two sampled (batch,
    K/V head) pairs, O and LSE of the group's 4 query heads, their dQ, and the K/V head's
    group-summed dK and dV, every element, against the oracle."""
    fa2 = _fa2()
    B, H, Hkv, N, d = 4, 16, 4, 2048, 128
    G = H // Hkv
    bq, bdo = normal_bf16((B, H, N, d), 9501), normal_bf16((B, H, N, d), 9504)
    bk, bv = normal_bf16((B, Hkv, N, d), 9502), normal_bf16((B, Hkv, N, d), 9503)
    q, k, v, do = (to_dev(b_) for b_ in (bq, bk, bv, bdo))
    o, lse = fa2.fwd(q, k, v, causal=True)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for b, kvh in ((0, 0), (3, 3)):
        hs = slice(kvh * G, (kvh + 1) * G)
        print(f"batch {b} K/V head {kvh}", flush=True)
        o_ref, lse_ref, dq_ref, dk_ref, dv_ref = _oracle(
            bq[b:b + 1, hs], bk[b:b + 1, kvh:kvh + 1], bv[b:b + 1, kvh:kvh + 1],
            bdo[b:b + 1, hs], True, default_scale(d))
        assert_fwd_close(bf16_to_f64(o[b:b + 1, hs]), lse[b:b + 1, hs].cpu().double().numpy(),
                         o_ref, lse_ref, f"b{b} kv{kvh}")
        for name, got, want in (("dq", dq[b:b + 1, hs], dq_ref),
                                ("dk", dk[b:b + 1, kvh:kvh + 1], dk_ref),
                                ("dv", dv[b:b + 1, kvh:kvh + 1], dv_ref)):
            assert_grad_close(bf16_to_f64(got), want, f"b{b} kv{kvh} {name}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_split_groups_match_whole_groups(d):
    """With the grouped workspace the dK/dV work of each group is split over several
    workgroups (fp32 partial sums added in a fixed order); with the plain workspace it is not.
    Both agree with the oracle, agree with each other to fp32 summation order, leave dQ
    unchanged, and the split path gives the same bits on a second run."""
    fa2 = _fa2()
    from exact_io_aware_42_amd import ops
    B, H, Hkv, N = 1, 8, 2, 300
    assert ops.bwd_workspace_bytes(B, H, N, d, Hkv) > ops.bwd_workspace_bytes(B, H, N, d)
    bq, bdo = normal_bf16((B, H, N, d), 9700 + d), normal_bf16((B, H, N, d), 9703 + d)
    bk, bv = normal_bf16((B, Hkv, N, d), 9701 + d), normal_bf16((B, Hkv, N, d), 9702 + d)
    q, k, v, do = (to_dev(b_) for b_ in (bq, bk, bv, bdo))
    o, lse = fa2.fwd(q, k, v, causal=True)
    g_split = fa2.bwd(q, k, v, o, do, lse, causal=True)
    g_split2 = fa2.bwd(q, k, v, o, do, lse, causal=True)
    small = torch.empty(ops.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    g_whole = fa2.bwd(q, k, v, o, do, lse, causal=True, workspace=small)
    torch.cuda.synchronize()
    for a_, b_ in zip(g_split, g_split2):
        assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
    assert torch.equal(g_split[0].view(torch.int16), g_whole[0].view(torch.int16))
    for a_, b_ in zip(g_split[1:], g_whole[1:]):
        torch.testing.assert_close(a_.float(), b_.float(), rtol=0,
                                   atol=1e-2 * b_.float().abs().max().item())
    _, _, dq_ref, dk_ref, dv_ref = _oracle(bq, bk, bv, bdo, True, default_scale(d))
    for name, got, want in (("dq", g_split[0], dq_ref), ("dk", g_split[1], dk_ref),
                            ("dv", g_split[2], dv_ref), ("dk whole", g_whole[1], dk_ref),
                            ("dv whole", g_whole[2], dv_ref)):
        assert_grad_close(bf16_to_f64(got), want, f"d{d} {name}")


SPLIT_CASES = [((1, 8, 1, 77, 64), True), ((1, 16, 2, 257, 128), False),
               ((2, 16, 16, 130, 128), True), ((1, 6, 3, 1, 256), True),
               ((1, 4, 4, 600, 256), False), ((3, 8, 8, 65, 64), True),
               ((1, 8, 8, 2048, 128), True), ((1, 8, 4, 2048, 64), False),
               ((4, 8, 4, 2048, 128), True), ((4, 8, 4, 2048, 128), False)]


@pytest.mark.parametrize("dims,causal", SPLIT_CASES,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-{'c' if c else 'f'}" for (b, h, hk, n, d), c in SPLIT_CASES])
def test_split_steps_match_oracle(dims, causal):
    """Small problems split each (key block, K/V head) pair's steps into parts (here 2, 4 and
    8, for one K/V head, many heads, a single query, ragged N, both masks; B4 H8 Hkv4 N2048
    d128 splits into 4 parts under the causal mask and 2 without): dQ, dK, dV against the
    oracle."""
    fa2 = _fa2()
    from exact_io_aware_42_amd import ops
    B, H, Hkv, N, d = dims
    assert ops.bwd_workspace_bytes(B, H, N, d, Hkv) > ops.bwd_workspace_bytes(B, H, N, d)
    seed = 9900 + H + N + d
    bq, bdo = normal_bf16((B, H, N, d), seed), normal_bf16((B, H, N, d), seed + 3)
    bk, bv = normal_bf16((B, Hkv, N, d), seed + 1), normal_bf16((B, Hkv, N, d), seed + 2)
    print(f"case {dims} causal={causal}", flush=True)
    q, k, v, do = (to_dev(b_) for b_ in (bq, bk, bv, bdo))
    o, lse = fa2.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa2.bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    _, _, dq_ref, dk_ref, dv_ref = _oracle(bq, bk, bv, bdo, causal, default_scale(d))
    if N == 1:
        # one key: P = 1, so dV is the sum of the group's dO and dQ = dK = 0 up to the rounding
        # of D = dO . O against dP = dO . V (the same products, summed in another order)
        assert_grad_close(bf16_to_f64(dv), dv_ref, f"{dims} dv")
        tiny = 1e-3 * np.abs(bf16_bits_to_f64(bdo)).max()
        assert np.abs(bf16_to_f64(dq)).max() <= tiny and np.abs(bf16_to_f64(dk)).max() <= tiny
        return
    for name, got, want in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        assert_grad_close(bf16_to_f64(got), want, f"{dims} {name}")
