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
                       (3, "FA2_ERR_HIP"), (4, "FA2_ERR_SCRATCH_LIMIT")):
        assert lib.fa2_status_string(code).decode() == name
    assert lib.fa2_last_hip_error() == 0


# Fake, 16-byte aligned, never dereferenced addresses: validation must fail before any use.
P = 0x10000


@pytest.mark.parametrize("args,expect", [
    ((None, P, P, P, P, 1, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),   # null q
    ((P, P, P, P, P + 4, 1, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),  # misaligned lse
    ((P, P, P, P, P, -1, 1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),     # B < 0
    ((P, P, P, P, P, 1, -1, 16, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),     # H < 0
    ((P, P, P, P, P, 1, 1, -5, 64, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),      # N < 0
    ((P, P, P, P, P, 1, 1, 16, 0, 0, 0.125), ops.FA2_ERR_INVALID_ARGUMENT),       # d = 0
    # empty problems are valid no-ops, even with null pointers (never examined)
    ((None, None, None, None, None, 0, 1, 16, 64, 0, 0.125), ops.FA2_OK),         # B = 0
    ((None, None, None, None, None, 2, 0, 16, 128, 1, 0.125), ops.FA2_OK),        # H = 0
    ((None, None, None, None, None, 1, 1, 0, 64, 1, 0.125), ops.FA2_OK),          # N = 0
    ((None, None, None, None, None, 1, 1, 0, 96, 0, 0.125), ops.FA2_ERR_UNSUPPORTED),
    ((None, None, None, None, None, 1, 1, 0, 64, 0, float("nan")), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, float("nan")), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, float("inf")), ops.FA2_ERR_INVALID_ARGUMENT),
    # any finite scale is accepted (0: uniform weights; < 0: reversed order), checked on
    # empty problems so that nothing is launched; |scale| * log2(e) must be a finite float
    ((None, None, None, None, None, 0, 1, 16, 64, 0, 0.0), ops.FA2_OK),
    ((None, None, None, None, None, 0, 1, 16, 64, 1, -0.5), ops.FA2_OK),
    ((None, None, None, None, None, 0, 1, 16, 64, 1, -3e38), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, 3e38), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 64, 0, float("-inf")), ops.FA2_ERR_INVALID_ARGUMENT),
    ((P, P, P, P, P, 1, 1, 16, 96, 0, 0.125), ops.FA2_ERR_UNSUPPORTED),           # d = 96
    ((P, P, P, P, P, 1, 1, 16, 512, 1, 0.125), ops.FA2_ERR_UNSUPPORTED),
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
    assert lib.fa2_bwd_workspace_bytes(2, 3, 0, 64) == 0
    assert lib.fa2_bwd_workspace_bytes(-1, 3, 10, 64) == 0
    # empty backward problems: no-ops that never look at the (null) pointers
    nul = [None] * 10
    assert lib.fa2_bwd(*nul, 0, 2, 3, 0, 64, 1, 0.125, None) == ops.FA2_OK
    assert lib.fa2_bwd_dq(*nul[:7], 0, None, 0, 3, 5, 128, 0, 0.125, None) == ops.FA2_OK
    assert lib.fa2_bwd_dkdv(*nul[:5], 0, None, None, 1, 0, 5, 64, 1, 0.125, None) == ops.FA2_OK
    assert lib.fa2_bwd_preprocess(*nul[:4], 0, 1, 1, 0, 64, None) == ops.FA2_OK
    assert lib.fa2_bwd_workspace_bytes(1, 1, 100, 80) == 0
    assert lib.fa2_bwd_workspace_bytes(1, 1, 100, 256) == 2 * 512
    assert lib.fa2_bwd_workspace_bytes(1, 1, 100, 512) == 0
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
    assert lib.fa2_bwd(*base, ws, 2, 3, 100, 320, 1, 0.125, None) == ops.FA2_ERR_UNSUPPORTED
    # stage entry points validate the same way
    assert lib.fa2_bwd_preprocess(P, P, P, P, ws - 1, 2, 3, 100, 64, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_preprocess(P, None, P, P, ws, 2, 3, 100, 64, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dkdv(P, P, P, P, P, ws, P, P, 2, 3, 100, 96, 1, 0.1, None) == \
        ops.FA2_ERR_UNSUPPORTED
    assert lib.fa2_bwd_dq(P, P, P, P, P, P, P, ws, None, 2, 3, 100, 64, 1, 0.1, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dq(P, P, P, P, P, P, P, ws, P, 2, 3, 100, 64, 1, 3e38, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dkdv(P, P, P, P, P, ws, P, P, 2, 3, 100, 64, 1, float("nan"), None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    # a negative or zero scale is valid (empty problem: nothing launched)
    assert lib.fa2_bwd(*nul, 0, 2, 3, 0, 64, 1, -0.125, None) == ops.FA2_OK
    assert lib.fa2_bwd(*nul, 0, 2, 3, 0, 64, 1, 0.0, None) == ops.FA2_OK
    assert lib.fa2_bwd_dq(P, P, P, None, P, P, P, ws, P, 2, 3, 100, 64, 1, 0.1, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT  # null o
    assert lib.fa2_bwd_dq(P, P, P, P, P, P + 4, P, ws, P, 2, 3, 100, 64, 1, 0.1, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT  # misaligned lse


HEAD_MAJOR, LONG_DESC, LONG_ASC = "head_major", "long_desc", "long_asc"


def schedule_tile_model(wg, n_blocks, bh_count, order, window=None):
    """Python model of the kernels' workgroup -> (block, batch*head) mapping; `window` heads per
    window of the causal orders (None: all of an XCD's heads)."""
    if bh_count % 8 == 0:
        xcd, j = wg % 8, wg // 8
        if order == HEAD_MAJOR:
            bh, r = (j // n_blocks) * 8 + xcd, j % n_blocks
        else:
            hpx = bh_count // 8
            win = hpx if window is None else window
            w, inner = divmod(j, win * n_blocks)
            wh = min(win, hpx - w * win)
            bh, r = (w * win + inner % wh) * 8 + xcd, inner // wh
    else:
        bh, r = wg % bh_count, wg // bh_count
    return (n_blocks - 1 - r if order == LONG_DESC else r), bh


def causal_work(qb, order, nq=16):
    """Relative length of block qb of nq: the forward/dQ block qb sees qb+1 key blocks, the
    dK/dV key block qb sees nq-qb query blocks."""
    return qb + 1 if order == LONG_DESC else nq - qb


@pytest.mark.parametrize("window", [None, 1, 2, 3])
@pytest.mark.parametrize("nq,bh", [(2, 2), (16, 256), (32, 64), (128, 16), (16, 64), (3, 5),
                                   (1, 8), (7, 24)])
@pytest.mark.parametrize("order", [HEAD_MAJOR, LONG_DESC, LONG_ASC])
def test_schedule_covers_every_tile_once(nq, bh, order, window):
    if window is not None and (order == HEAD_MAJOR or bh % 8 or window > bh // 8):
        pytest.skip("window applies to the causal orders with whole heads per XCD")
    seen = set()
    for wg in range(nq * bh):
        qb, h = schedule_tile_model(wg, nq, bh, order, window)
        assert 0 <= qb < nq and 0 <= h < bh
        seen.add((qb, h))
    assert len(seen) == nq * bh
    if bh % 8 == 0:
        # every head's blocks run on one XCD (workgroup id mod 8)
        for wg in range(nq * bh):
            assert schedule_tile_model(wg, nq, bh, order, window)[1] % 8 == wg % 8
    if order != HEAD_MAJOR and bh % 8 == 0:
        # per XCD, each window's blocks come in non-increasing length order over its heads
        hpx = bh // 8
        win = hpx if window is None else window
        for x in range(8):
            seq = [schedule_tile_model(wg, nq, bh, order, window) for wg in range(x, nq * bh, 8)]
            for w0 in range(0, len(seq), win * nq):
                part = seq[w0:w0 + win * nq]
                assert len({h // 8 // win for _, h in part}) == 1  # one window at a time
                lens = [causal_work(qb, order, nq) for qb, _ in part]
                assert lens == sorted(lens, reverse=True)


def _makespan(order, nq=16, bh=64, slots=64, window=None):
    """Greedy list schedule of one XCD's blocks on `slots` workgroup slots."""
    import heapq
    free = [0.0] * slots
    for wg in range(0, nq * bh, 8):
        qb, _ = schedule_tile_model(wg, nq, bh, order, window)
        t = heapq.heappop(free)
        heapq.heappush(free, t + causal_work(qb, LONG_DESC, nq))
    return max(free)


def test_longest_first_shortens_the_causal_tail():
    """For the causal forward with 8 heads per XCD, dealing the blocks longest first ends within
    a few percent of the ideal (total work / slots); head by head it does not."""
    total = 8 * sum(range(1, 17))
    ideal = total / 64
    assert _makespan(LONG_DESC) <= 1.15 * ideal
    assert _makespan(LONG_DESC, window=4) <= 1.15 * ideal
    assert _makespan(LONG_DESC) < _makespan(HEAD_MAJOR)


def _l2_model(order, nq, bh, window, slots, tile_bytes, tiles_of, first_of, cap=4 << 20):
    """One XCD (workgroup id % 8 == 0): its blocks run as a list schedule on `slots` workgroup
    slots, every block reading its head's streamed tiles first_of(qb) .. + tiles_of(qb) - 1 in
    order, one tile per time step; an LRU cache of `cap` bytes at tile granularity stands for
    the XCD's L2. Returns (makespan / ideal, tile bytes fetched / compulsory bytes)."""
    from collections import OrderedDict
    queue = [schedule_tile_model(wg, nq, bh, order, window) for wg in range(0, nq * bh, 8)]
    queue.reverse()
    cache, active, misses, t = OrderedDict(), [], 0, 0
    while queue or active:
        while len(active) < slots and queue:
            qb, h = queue.pop()
            active.append([h, first_of(qb), first_of(qb) + tiles_of(qb)])
        nxt = []
        for blk in active:
            key = (blk[0], blk[1])
            if key in cache:
                cache.move_to_end(key)
            else:
                misses += 1
                cache[key] = True
                if len(cache) * tile_bytes > cap:
                    cache.popitem(last=False)
            blk[1] += 1
            if blk[1] < blk[2]:
                nxt.append(blk)
        active, t = nxt, t + 1
    heads = bh // 8
    ideal = heads * sum(tiles_of(b) for b in range(nq)) / slots
    compulsory = heads * max(first_of(b) + tiles_of(b) for b in range(nq))
    return t / ideal, misses / compulsory


# (kernel and workload, order, blocks per head, heads, window of 4 MiB of streamed tiles, slots
#  per XCD, streamed tile bytes, tiles of block qb, first tile of block qb). causal_window()
#  gives these windows for a 4 MiB budget (pinned in tests/abi_host_check.cpp).
L2_CASES = [
    ("fwd B8 H32 N2048 d64", LONG_DESC, 16, 256, 8, 96, 16 << 10, lambda b: 2 * (b + 1), lambda b: 0),
    ("fwd B4 H16 N4096 d128", LONG_DESC, 16, 64, 2, 32, 32 << 10, lambda b: 4 * (b + 1), lambda b: 0),
    ("fwd B1 H16 N16384 d128", LONG_DESC, 64, 16, 1, 32, 32 << 10, lambda b: 4 * (b + 1), lambda b: 0),
    ("dQ B4 H16 N2048 d128", LONG_DESC, 8, 64, 4, 32, 32 << 10, lambda b: 4 * (b + 1), lambda b: 0),
    ("dK/dV B4 H16 N2048 d128", LONG_ASC, 16, 64, 4, 32, 32 << 10, lambda b: 32 - 2 * b,
     lambda b: 2 * b),
]


@pytest.mark.parametrize("case", L2_CASES, ids=[c[0] for c in L2_CASES])
def test_causal_windows_keep_the_l2_working_set(case):
    """Modelled on one XCD: windows of heads whose streamed tiles fit 4 MiB fetch each tile
    about once and end within 10% of the ideal makespan; dealing all of an XCD's heads at once
    refetches tiles whenever more than one window's heads are in flight."""
    name, order, nq, bh, window, slots, tb, tiles_of, first_of = case
    span, traffic = _l2_model(order, nq, bh, window, slots, tb, tiles_of, first_of)
    span_all, traffic_all = _l2_model(order, nq, bh, None, slots, tb, tiles_of, first_of)
    print(f"{name}: window {window}: makespan {span:.3f}x ideal, traffic {traffic:.2f}x; "
          f"all heads: {span_all:.3f}x, {traffic_all:.2f}x")
    # one head's K/V at N = 16384, d = 128 is 8 MiB, twice the L2: blocks of that one head in
    # flight already refetch some tiles
    limit = 1.6 if "N16384" in name else 1.10
    assert span <= 1.10 and traffic <= limit
    if bh // 8 > window:
        assert traffic_all > 1.4


def test_host_window_at_d64():
    """The host's choice at d = 64 (an 8 MiB budget: windows of 16 of the 32 heads per XCD at
    B8 H32 N2048, three forward workgroups per CU), which measured fastest on the GPU: in the
    model it ends within 5% of the ideal and fetches well under the all-heads deal."""
    name, order, nq, bh, _, slots, tb, tiles_of, first_of = L2_CASES[0]
    span, traffic = _l2_model(order, nq, bh, 16, slots, tb, tiles_of, first_of)
    _, traffic_all = _l2_model(order, nq, bh, None, slots, tb, tiles_of, first_of)
    assert span <= 1.05 and traffic <= 0.65 * traffic_all


def test_grouped_kv_validation():
    """fa2_fwd_gqa / fa2_bwd_gqa reject bad K/V head counts and strides before any HIP call
    (the pointers are fake; every case has an invalid parameter)."""
    lib = _lib()
    N, d = 16, 64
    ok = dict(B=2, H=8, Hkv=2, kvs=2 * N * d)
    def fwd(B=2, H=8, Hkv=2, kvs=2 * N * d, d_=d):
        return lib.fa2_fwd_gqa(P, P, P, P, P, B, H, Hkv, N, d_, kvs, 1, 0.125, None)
    assert fwd(Hkv=3) == ops.FA2_ERR_INVALID_ARGUMENT            # 8 % 3 != 0
    assert fwd(Hkv=0) == ops.FA2_ERR_INVALID_ARGUMENT
    assert fwd(Hkv=16) == ops.FA2_ERR_INVALID_ARGUMENT           # more K/V heads than Q heads
    assert fwd(kvs=2 * N * d - 8) == ops.FA2_ERR_INVALID_ARGUMENT  # batches overlap
    assert fwd(kvs=2 * N * d + 4) == ops.FA2_ERR_INVALID_ARGUMENT  # not a multiple of 8
    assert fwd(Hkv=3, d_=96) == ops.FA2_ERR_UNSUPPORTED
    ws = lib.fa2_bwd_workspace_bytes(2, 8, N, d)
    base = [P] * 10
    assert lib.fa2_bwd_gqa(*base, ws, 2, 8, 3, N, d, 3 * N * d, 0, 0.125, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_gqa(*base, ws, 2, 8, 2, N, d, N * d, 0, 0.125, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_gqa(*base, ws - 1, 2, 8, 2, N, d, 2 * N * d, 0, 0.125, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    # empty problems stay no-ops
    assert lib.fa2_fwd_gqa(None, None, None, None, None, 0, 8, 2, N, d, 2 * N * d, 1, 0.125,
                           None) == ops.FA2_OK


def test_dropout_validation():
    """fa2_fwd_dropout / fa2_bwd_dropout reject a probability outside [0, 1) (NaN included)
    before any HIP call; the pointers are fake and every case has an invalid parameter."""
    lib = _lib()
    N, d = 16, 64
    ws = lib.fa2_bwd_workspace_bytes(2, 8, N, d)
    for p in (1.0, 1.5, -0.1, float("nan"), float("inf")):
        assert lib.fa2_fwd_dropout(P, P, P, P, P, 2, 8, 2, N, d, 2 * N * d, 1, 0.125, p, 1, 2,
                                   None) == ops.FA2_ERR_INVALID_ARGUMENT, p
        assert lib.fa2_bwd_dropout(*([P] * 10), ws, 2, 8, 2, N, d, 2 * N * d, 0, 0.125, p, 1,
                                   2, None) == ops.FA2_ERR_INVALID_ARGUMENT, p
    # a valid probability does not excuse other invalid arguments
    assert lib.fa2_fwd_dropout(P, P, P, P, P, 2, 8, 3, N, d, 3 * N * d, 1, 0.125, 0.1, 1, 2,
                               None) == ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_fwd_dropout(None, P, P, P, P, 2, 8, 2, N, d, 2 * N * d, 1, 0.125, 0.1, 1, 2,
                               None) == ops.FA2_ERR_INVALID_ARGUMENT
    assert lib.fa2_bwd_dropout(*([P] * 10), ws - 1, 2, 8, 2, N, d, 2 * N * d, 0, 0.125, 0.1, 1,
                               2, None) == ops.FA2_ERR_INVALID_ARGUMENT
    # empty problems stay no-ops
    assert lib.fa2_fwd_dropout(None, None, None, None, None, 2, 8, 2, 0, d, 0, 1, 0.125, 0.5, 1,
                               2, None) == ops.FA2_OK


def _split_model(B, H, Hkv, N, d, causal=True):
    """The rule the backward uses: split each (key block, K/V head) pair's steps only while
    those pairs number under the target (1024 workgroups under the causal mask, 512 without),
    into the smallest count from 2 to 8 that reaches it (else 8); key blocks of 64 at d = 256,
    128 otherwise. The workspace size follows the causal rule (the larger split)."""
    kb = -(-N // (64 if d == 256 else 128))
    base = kb * B * Hkv
    target = 1024 if causal else 512
    if base >= target:
        return 1
    for s in range(2, 8):
        if base * s >= target:
            return s
    return 8


@pytest.mark.parametrize("B,H,Hkv,N,d", [(4, 16, 4, 2048, 128), (1, 32, 4, 2048, 128),
                                         (8, 32, 8, 4096, 128), (2, 8, 2, 150, 64),
                                         (1, 64, 8, 4096, 256), (2, 12, 4, 1000, 64),
                                         (3, 6, 6, 700, 128), (1, 8, 1, 64, 128),
                                         (1, 8, 8, 2048, 128), (4, 16, 16, 2048, 128)])
def test_grouped_workspace_size(B, H, Hkv, N, d):
    """fa2_bwd_gqa_workspace_bytes = the plain workspace plus 2 * parts * B*Hkv*N*d fp32
    partial sums (rounded up to 256 bytes) when the dK/dV work is split (Hkv = H included)."""
    lib = _lib()
    base = lib.fa2_bwd_workspace_bytes(B, H, N, d)
    s = _split_model(B, H, Hkv, N, d)
    extra = 0 if s == 1 else -(-(2 * s * B * Hkv * N * d * 4) // 256) * 256
    assert lib.fa2_bwd_gqa_workspace_bytes(B, H, Hkv, N, d) == base + extra
    assert ops.bwd_workspace_bytes(B, H, N, d, Hkv) == base + extra


def test_grouped_workspace_size_invalid():
    lib = _lib()
    assert lib.fa2_bwd_gqa_workspace_bytes(2, 8, 3, 64, 128) == 0   # 3 does not divide 8
    assert lib.fa2_bwd_gqa_workspace_bytes(2, 8, 0, 64, 128) == 0
    assert lib.fa2_bwd_gqa_workspace_bytes(2, 8, 2, 0, 128) == 0    # empty
    assert lib.fa2_bwd_gqa_workspace_bytes(2, 8, 2, 64, 96) == 0    # unsupported d


def test_noalloc_validation_and_limit():
    """fa2_bwd_noalloc validates like fa2_bwd and refuses problems beyond its static scratch
    (B*H*N rows above fa2_bwd_noalloc_max_rows) before any HIP call."""
    lib = _lib()
    max_rows = lib.fa2_bwd_noalloc_max_rows()
    assert max_rows == 1 << 21
    nul = [None] * 9
    assert lib.fa2_bwd_noalloc(*nul, 0, 2, 3, 64, 1, 0.125, None) == ops.FA2_OK  # empty
    base = [P] * 9
    assert lib.fa2_bwd_noalloc(*base, 2, 3, 100, 96, 1, 0.125, None) == ops.FA2_ERR_UNSUPPORTED
    assert lib.fa2_bwd_noalloc(*base, 2, 3, 100, 64, 1, float("nan"), None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    args = list(base)
    args[6] = None  # null dq
    assert lib.fa2_bwd_noalloc(*args, 2, 3, 100, 64, 1, 0.125, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    args = list(base)
    args[5] = P + 4  # misaligned lse
    assert lib.fa2_bwd_noalloc(*args, 2, 3, 100, 64, 1, 0.125, None) == \
        ops.FA2_ERR_INVALID_ARGUMENT
    # one row past the limit: B*H*N = 2^21 + 1 (as 1 x 1 x N), and a larger batch
    assert lib.fa2_bwd_noalloc(*base, 1, 1, max_rows + 1, 64, 0, 0.125, None) == \
        ops.FA2_ERR_SCRATCH_LIMIT
    assert lib.fa2_bwd_noalloc(*base, 8, 32, 16384, 128, 1, 0.125, None) == \
        ops.FA2_ERR_SCRATCH_LIMIT
