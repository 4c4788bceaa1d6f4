"""CPU-only checks of the C ABI: libfa2.so loads, exports every symbol include/fa2.h
declares, and rejects invalid arguments on the host before any HIP call (these calls never
reach a kernel launch, so no GPU is needed). Also a pure-Python model of the workgroup
schedule (the same formula the kernels use) is checked for exact coverage."""
import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_42_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def _lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libfa2.so not built")
    return ops.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fa2_status|size_t|const char\*|int)\s+(fa2_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_abi():
    assert _declared() == sorted(ops.EXPORTED)


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa2_\w+)", out))
    for name in _declared():
        assert name in exported, name


def test_status_strings():
    lib = _lib()
    for code, name in ((0, "FA2_OK"), (1, "FA2_ERR_INVALID_ARGUMENT"), (2, "FA2_ERR_UNSUPPORTED"),
                       (3, "FA2_ERR_HIP")):
        assert lib.fa2_status_string(code).decode() == name
    assert lib.fa2_last_hip_error() == 0


# Fake, 16-byte aligned, never dereferenced addresses: validation must fail before any use.
P = 0x10000


@pytest.mark.parametrize("args,expect", [
    ((None, P, P, P, P, 1, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),   # null q
    ((P, P, P, P, P + 4, 1, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),  # misaligned lse
    ((P, P, P, P, P, 0, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),      # B = 0
    ((P, P, P, P, P, 1, -1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),     # H < 0
    ((P, P, P, P, P, 1, 1, 0, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),       # N = 0
    ((P, P, P, P, P, 1, 1, 16, 64, 0, float("nan")), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, float("inf")), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, 0.0), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, -0.5), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 96, 0, 0.125), ops.FA2_ERR_UNSUPPORTED),           # d = 96
    ((P, P, P, P, P, 1, 1, 16, 256, 1, 0.125), ops.FA2_ERR_UNSUPPORTED),
    ((P, P, P, P, P, 1 << 20, 1 << 10, 1 << 20, 128, 0, 0.1), ops.FA2_ERR_INVALID_ARGUMENT),
])
def test_fwd_validation(args, expect):
    lib = _lib()
    assert lib.fa2_fwd(*args, None) == expect


def test_bwd_validation_and_workspace():
    lib = _lib()
    ws = lib.fa2_bwd_workspace_bytes(2, 3, 100, 64)
    assert ws >= 2 * (2 * 3 * 100 * 4) and ws % 256 == 0
    assert lib.fa2_bwd_workspace_bytes(0, 3, 100, 64) == 0
    assert lib.fa2_bwd_workspace_bytes(1, 1, 100, 80) == 0
    base = [P] * 10
    ok_sizes = (2, 3, 100, 64, 1, 0.125)
    # workspace too small
    assert lib.fa2_bwd(*base, ws - 1, *ok_sizes, None) == ops.FA2_ERR_INVALID_ARGUMENT
    # null dk
    args = list(base)
    args[7] = None
    assert lib.fa2_bwd(*args, ws, *ok_sizes, None) == ops.FA2_ERR_INVALID_ARGUMENT
    # misaligned workspace
    args = list(base)
    args[9] = P + 8
    assert lib.fa2_bwd(*args, ws, *ok_sizes, None) == ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd(*base, ws, 2, 3, 100, 48, 1, 0.125, None) == ops.FA2_ERR_UNSUPPORTED
    # stage entry points validate the same way
    assert lib.fa2_bwd_preprocess(P, P, P, P, ws - 1, 2, 3, 100, 64, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_preprocess(P, None, P, P, ws, 2, 3, 100, 64, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dkdv(P, P, P, P, P, ws, P, P, 2, 3, 100, 96, 1, 0.1, None) == \
        ops.FA2_ERR_UNSUPPORTED
    assert lib.fa2_bwd_dq(P, P, P, P, P, ws, None, 2, 3, 100, 64, 1, 0.1, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dq(P, P, P, P, P, ws, P, 2, 3, 100, 64, 1, -1.0, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT


def schedule_tile_model(wg, n_qblocks, bh_count, heavy_first):
    """Python model of the kernels' workgroup -> (query block, batch*head) mapping."""
    if bh_count % 8 == 0:
        xcd, j = wg % 8, wg // 8
        bh = (j // n_qblocks) * 8 + xcd
        qr = j % n_qblocks
    else:
        bh, qr = wg % bh_count, wg // bh_count
    return (n_qblocks - 1 - qr if heavy_first else qr), bh


@pytest.mark.parametrize("nq,bh", [(2, 2), (16, 256), (32, 64), (128, 16), (16, 64), (3, 5),
                                   (1, 8), (7, 24)])
@pytest.mark.parametrize("heavy", [False, True])
def test_schedule_covers_every_tile_once(nq, bh, heavy):
    seen = set()
    for wg in range(nq * bh):
        qb, h = schedule_tile_model(wg, nq, bh, heavy)
        assert 0 <= qb < nq and 0 <= h < bh
        seen.add((qb, h))
    assert len(seen) == nq * bh
    if bh % 8 == 0:
        # every head's query blocks run on one XCD (workgroup id mod 8)
        for wg in range(nq * bh):
            assert schedule_tile_model(wg, nq, bh, heavy)[1] % 8 == wg % 8
    if heavy:
        # per XCD, a head's blocks start with the longest (highest index) one
        firsts = {}
        for wg in range(nq * bh):
            qb, h = schedule_tile_model(wg, nq, bh, heavy)
            firsts.setdefault(h, qb)
        assert all(v == nq - 1 for v in firsts.values())
