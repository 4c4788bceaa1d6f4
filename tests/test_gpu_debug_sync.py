"""Race check: the FA2_DEBUG_SYNC build (libfa2_debug_sync.so: the same sources with every wave
waiting for all of its loads and the workgroup meeting at a barrier at each LDS stage
hand-over) must give the normal build's results bit for bit. A missing wait or barrier in the
normal build, which lets a tile be read before it has landed or be refilled while still read,
would make the two differ. Both builds are called through the C ABI on the same inputs:
forward, backward (minimum workspace and the split dK/dV path), grouped K/V heads and
dropout, d = 64, 128, 256, both masks, ragged N."""
import ctypes
import os

import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import default_scale, normal_bf16

from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "exact_io_aware_42_amd")


def _libs():
    import exact_io_aware_42_amd as fa2
    from exact_io_aware_42_amd.ops import open_library
    return fa2.load_library(), open_library(os.path.join(PKG, "libfa2_debug_sync.so"))


def _run(lib, q, k, v, do, B, H, Hkv, N, d, causal, p, split):
    dev = q.device
    scale = default_scale(d)
    stream = torch.cuda.current_stream().cuda_stream
    kvs = Hkv * N * d
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    st = lib.fa2_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, Hkv, N, d, kvs, int(causal), scale, p, 5, 6,
                             stream)
    assert st == 0
    ws_bytes = (lib.fa2_bwd_gqa_workspace_bytes(B, H, Hkv, N, d) if split
                else lib.fa2_bwd_workspace_bytes(B, H, N, d))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    st = lib.fa2_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), ws.data_ptr(), ctypes.c_size_t(ws_bytes), B, H, Hkv,
                             N, d, kvs, int(causal), scale, p, 5, 6, stream)
    assert st == 0
    torch.cuda.synchronize()
    return [bits_of(o), lse.view(torch.int32).cpu().numpy(), bits_of(dq), bits_of(dk),
            bits_of(dv)]


CASES = [  # B, H, Hkv, N, d, causal, dropout p, split dK/dV
    (2, 4, 4, 1000, 128, True, 0.0, False), (2, 4, 4, 1000, 128, False, 0.0, True),
    (1, 8, 2, 777, 64, True, 0.0, True), (3, 2, 2, 513, 64, False, 0.1, False),
    (1, 4, 4, 700, 256, True, 0.0, False), (2, 2, 1, 333, 256, False, 0.2, True),
    (4, 16, 16, 2048, 128, True, 0.0, False),  # the fwd+bwd workload's shape
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}/{c[2]}x{c[3]}x{c[4]}"
                                             f"-{'c' if c[5] else 'f'}-p{c[6]}"
                                             f"{'-split' if c[7] else ''}" for c in CASES])
def test_debug_sync_build_is_bit_identical(case):
    B, H, Hkv, N, d, causal, p, split = case
    print(f"case {case}", flush=True)
    lib, dbg = _libs()
    seed = 9100 + N + d
    q, do = to_dev(normal_bf16((B, H, N, d), seed)), to_dev(normal_bf16((B, H, N, d), seed + 1))
    k, v = (to_dev(normal_bf16((B, Hkv, N, d), seed + 2 + t)) for t in range(2))
    a = _run(lib, q, k, v, do, B, H, Hkv, N, d, causal, p, split)
    b = _run(dbg, q, k, v, do, B, H, Hkv, N, d, causal, p, split)
    for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), a, b):
        np.testing.assert_array_equal(x, y, err_msg=f"{case} {name}")
