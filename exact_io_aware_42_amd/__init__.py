"""FlashAttention-2 exact attention for MI355X (gfx950): HIP kernels behind a C ABI
(include/fa2.h, libfa2.so) and a thin ctypes binding.

    from exact_io_aware_42_amd import fwd, bwd
    o, lse = fwd(q, k, v, causal=True)            # bf16 [B, H, N, d] on the GPU
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True)

    from exact_io_aware_42_amd import flash_attn_func
    o = flash_attn_func(q, k, v, causal=True)     # differentiable (torch.autograd)

The library is loaded on first use; if it has not been built the call raises (there is no
fallback path).
"""
from .autograd import (FlashAttention, FlashAttentionKVPacked, flash_attn_func,
                       flash_attn_kvpacked_func)
from .ops import (FA2Error, bwd, bwd_dkdv, bwd_dq, bwd_kvpacked, bwd_noalloc,
                  bwd_noalloc_max_rows, bwd_preprocess, bwd_workspace_bytes, fwd, fwd_kvpacked,
                  load_library)

__all__ = ["fwd", "bwd", "fwd_kvpacked", "bwd_kvpacked", "bwd_preprocess", "bwd_dkdv", "bwd_dq",
           "bwd_noalloc", "bwd_noalloc_max_rows", "bwd_workspace_bytes", "load_library", "FA2Error", "FlashAttention",
           "FlashAttentionKVPacked", "flash_attn_func", "flash_attn_kvpacked_func"]
