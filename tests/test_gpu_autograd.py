"""The torch.autograd face (`flash_attn_func`) and the GPT-style layer harness on the GPU.

Gradients through autograd are compared with the CPU float64 oracle (same bound as the
backward tests: max|g - g_ref| <= 2e-2 * max|g_ref|) and, bit for bit, with direct fwd/bwd
calls. The layer test captures the layer's own q, k, v and attention cotangent and checks the
attention gradients it received against the oracle, and checks the whole layer against a
float64 CPU layer built from the same bf16 parameters (projections in bf16 add their own
rounding there, so that bound is looser and derived below).
"""
import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import bf16_bits_to_f64, default_scale, normal_bf16
from oracle import attention_backward, attention_forward

from gpu_util import assert_grad_close, bf16_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _fa2():
    import exact_io_aware_42_amd as fa2
    return fa2


@pytest.mark.parametrize("shape,causal", [((1, 2, 150, 64), True), ((2, 1, 97, 128), False),
                                          ((1, 1, 70, 256), True)])
def test_autograd_matches_oracle_and_direct_calls(shape, causal):
    fa2 = _fa2()
    bq, bk, bv, bdo = (normal_bf16(shape, 9100 + t) for t in range(4))
    q, k, v = (to_dev(b).requires_grad_() for b in (bq, bk, bv))
    do = to_dev(bdo)
    o = fa2.flash_attn_func(q, k, v, causal=causal)
    o.backward(do)
    torch.cuda.synchronize()
    scale = default_scale(shape[3])
    ref = attention_backward(*(bf16_bits_to_f64(b) for b in (bq, bk, bv, bdo)), causal=causal,
                             scale=scale)
    for name, t, want in zip(("dq", "dk", "dv"), (q, k, v), ref):
        assert_grad_close(bf16_to_f64(t.grad), want, f"autograd {name}")
    o2, lse2 = fa2.fwd(q.detach(), k.detach(), v.detach(), causal=causal)
    g2 = fa2.bwd(q.detach(), k.detach(), v.detach(), o2, do, lse2, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach().view(torch.int16), o2.view(torch.int16))
    for t, g in zip((q, k, v), g2):
        assert torch.equal(t.grad.view(torch.int16), g.view(torch.int16))


def _layer_f64(x, w_qkv, w_o, dy, H):
    """The same layer in float64 on the CPU (explicit softmax attention), with autograd."""
    x, w_qkv, w_o = (t.detach().cpu().double().requires_grad_() for t in (x, w_qkv, w_o))
    B, N, C = x.shape
    d = C // H
    qkv = (x @ w_qkv).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4)
    q, k, v = qkv[0], qkv[1], qkv[2]
    s = (q @ k.transpose(-1, -2)) * float(default_scale(d))
    s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ v
    y = o.permute(0, 2, 1, 3).reshape(B, N, C) @ w_o
    y.backward(dy.detach().cpu().double())
    return y.detach(), x.grad, w_qkv.grad, w_o.grad


def test_gpt_layer_step():
    from exact_io_aware_42_amd.gpt_layer import layer_forward, make_params
    B, N, H, d = 2, 200, 2, 64
    dev = torch.device("cuda:0")
    x, w_qkv, w_o, dy = make_params(B, N, H, d, dev, seed=3)
    keep = {}
    y = layer_forward(x, w_qkv, w_o, H, keep=keep)
    grads = {}
    for name in ("q", "k", "v"):
        keep[name].register_hook(lambda g, name=name: grads.__setitem__(name, g))
    keep["o"].register_hook(lambda g: grads.__setitem__("o", g))
    y.backward(dy)
    torch.cuda.synchronize()
    # 1. the attention gradients the layer received, against the oracle on the layer's own
    #    bf16 q, k, v and attention cotangent
    q64, k64, v64, do64 = (bf16_to_f64(t.detach()) for t in
                           (keep["q"], keep["k"], keep["v"], grads["o"]))
    scale = default_scale(d)
    o_ref, _ = attention_forward(q64, k64, v64, causal=True, scale=scale)
    assert np.abs(bf16_to_f64(keep["o"].detach()) - o_ref).max() <= 1e-2
    ref = attention_backward(q64, k64, v64, do64, causal=True, scale=scale)
    for name, want in zip(("q", "k", "v"), ref):
        assert_grad_close(bf16_to_f64(grads[name]), want, f"layer d{name}")
    # 2. the whole layer against float64: bf16 rounding of the stored activations (qkv, o, y)
    #    and of the gradients between the matmuls (about 2^-8 relative each, a few stages
    #    deep) gives a bound of 5e-2 of the largest entry
    y64, gx, gw, go = _layer_f64(x, w_qkv, w_o, dy, H)
    for name, got, want in (("y", y, y64), ("dx", x.grad, gx), ("dW_qkv", w_qkv.grad, gw),
                            ("dW_o", w_o.grad, go)):
        got = got.detach().double().cpu().numpy()
        want = want.numpy()
        err = np.abs(got - want).max() / np.abs(want).max()
        assert err <= 5e-2, f"{name}: relative error {err:.3g}"
