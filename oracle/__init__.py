"""CPU float64 oracle for exact attention and its gradients.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check (`__graft_entry__.smoke`) and the
benchmark's CPU-baseline leg may import this package. The HIP library and its Python
binding share no code with it and never call it.

Modules:
  attention   plain definition: forward (O, LSE), probabilities, analytic backward (whole,
              or at sampled query rows and key rows)
  bruteforce  scalar loops for tiny shapes
  online      float64 model of the tiled online-softmax recurrence
  dropout     attention with dropout on P and its counter-based mask generator

Every function here is pinned by CPU tests to something other than itself (brute force,
closed forms, invariants, finite differences, PyTorch's CPU scaled_dot_product_attention,
hand-derived values under tests/golden/).
"""
from .attention import (attention_backward, attention_backward_sampled, attention_forward,
                        attention_probs, resolve_scale)
from .bruteforce import attention_bruteforce
from .dropout import (attention_backward_dropout, attention_backward_dropout_sampled,
                      attention_forward_dropout, keep_mask, keep_scale, pcg_hash)
from .online import online_attention_forward

__all__ = [
    "attention_forward",
    "attention_backward",
    "attention_backward_sampled",
    "attention_probs",
    "resolve_scale",
    "attention_bruteforce",
    "online_attention_forward",
    "attention_forward_dropout",
    "attention_backward_dropout_sampled",
    "attention_backward_dropout",
    "keep_mask",
    "keep_scale",
    "pcg_hash",
]
