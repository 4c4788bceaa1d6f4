"""The forward and the no-allocation backward (fa2_bwd_noalloc) captured in one HIP graph and
replayed: every replay must reproduce the eager results bit for bit. Between replays the
program runs eager work of its own (outputs refilled with NaN, and an eager no-allocation
backward of another shape that overwrites the shared scratch array), with synchronisations
in between, so a replay can neither lean on values left by the previous one nor on the
scratch contents at capture time."""
import numpy as np
import pytest
import torch

from exact_io_aware_42_amd.inputs import default_scale, normal_bf16

from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu


def _nan_like(t):
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("causal", [True, False])
def test_graph_replays_match_eager(causal):
    import exact_io_aware_42_amd as fa2
    shape = (2, 4, 640, 128)   # several query tiles and key blocks per head
    print(f"graph capture fwd+bwd_noalloc {shape} causal={causal}", flush=True)
    scale = default_scale(shape[-1])
    q, k, v, do = (to_dev(normal_bf16(shape, 950 + t)) for t in range(4))

    # eager results; the first no-allocation call also looks up the scratch array's address,
    # which is not a stream operation and so stays out of the capture
    o_ref, lse_ref = fa2.fwd(q, k, v, causal=causal, scale=scale)
    g_ref = fa2.bwd_noalloc(q, k, v, o_ref, do, lse_ref,
                            *(_nan_like(q) for _ in range(3)), causal=causal, scale=scale)
    torch.cuda.synchronize()

    # other eager work that uses the same scratch array between replays
    other = (1, 3, 333, 64)
    q2, k2, v2, do2 = (to_dev(normal_bf16(other, 960 + t)) for t in range(4))
    o2, lse2 = fa2.fwd(q2, k2, v2, causal=not causal)
    g2 = [torch.empty_like(q2) for _ in range(3)]

    o = _nan_like(o_ref)
    lse = _nan_like(lse_ref)
    g = [_nan_like(q) for _ in range(3)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa2.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        fa2.bwd_noalloc(q, k, v, o, do, lse, *g, causal=causal, scale=scale)
    torch.cuda.synchronize()

    for replay in range(3):
        for t in (o, lse, *g):
            t.fill_(float("nan"))
        fa2.bwd_noalloc(q2, k2, v2, o2, do2, lse2, *g2, causal=not causal)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in (("o", o, o_ref), ("lse", lse, lse_ref),
                               ("dq", g[0], g_ref[0]), ("dk", g[1], g_ref[1]),
                               ("dv", g[2], g_ref[2])):
            assert torch.isfinite(got.float()).all(), f"replay {replay} {name}"
            np.testing.assert_array_equal(bits_of(got), bits_of(ref),
                                          err_msg=f"replay {replay} {name}")
    del graph
