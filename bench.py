"""Benchmark: FlashAttention-2 forward + backward on one MI355X through the fa2 C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--direction both]

One step is one pass of the whole hot path over one batch of synthetic seeded inputs
(i.i.d. N(0, 1) bf16, already resident in device memory): the forward kernel (O and LSE)
and the backward (the dQ kernel, which also forms D = rowsum(dO * O), then the dK/dV kernel). The default workload
is the fwd+bwd attention workload B=4, H=16, N=2048, d=128, causal. FLOP counts: forward
4*B*H*N^2*d (halved when causal), backward 2.5x forward. `value` is the step's total FLOP
over its wall time, in TFLOP/s.

Each kernel launch in the timed region is bracketed by HIP events on the stream it runs on;
the `roofline` object describes the kernel with the largest share of the step time:
achieved = its algorithmic FLOP per launch / its mean event-measured duration, against the
dense bf16 MFMA peak of MI355X (2.5 PFLOP/s). `traffic` comes from committed rocprofv3
FETCH_SIZE / WRITE_SIZE counter summaries under profiles/ (null if the kernel source changed
since they were taken). `cpu_baseline` times the CPU float64 oracle on a bounded sample of
the same workload (whole heads) on the host cores. `forward_workloads` adds the forward
kernel's TFLOP/s on the forward-only workloads, `non_causal_step` the same fwd+bwd step
without the causal mask, `d256_steps` the fwd+bwd step at head dimension 256, `gpt_layer_step` a GPT-style attention layer (bf16 projections + attention,
forward and backward through torch.autograd), `gqa_step` the fwd+bwd step with 16 query
heads sharing 4 K/V heads, `dropout_step` the fwd+bwd step with dropout p = 0.1 on the
attention probabilities, `graph_step` the fwd+bwd step captured in a HIP graph and replayed,
and `gemm_yardstick` a library bf16 GEMM (8192^3, torch.matmul) on the same chip, for context;
none of them is part of `value`.

Prints ONE JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
WARM_MS = 300.0  # GPU time of untimed steps before the counted warm-up
METRIC = "attention fwd/bwd TFLOP/s (bf16, causal+non-causal) and % of MFMA peak, 1 GPU"


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--causal", choices=("default", "causal", "full"), default="default")
    ap.add_argument("--direction", choices=("both", "fwd"), default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fwd-sweep", action="store_true",
                    help="skip the forward-only timing of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget for the oracle baseline sample")
    return ap.parse_args()


def fwd_flop(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def cpu_baseline(w, causal, with_bwd, budget_s):
    """Time the CPU float64 oracle on whole (batch, head) slices of the same inputs until the
    budget is spent; scale to TFLOP/s with the same FLOP formula."""
    import numpy as np

    from exact_io_aware_42_amd.inputs import bf16_bits_to_f64, default_scale, workload_tensors
    from oracle import attention_backward, attention_forward

    from threadpoolctl import threadpool_info

    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max([p.get("num_threads", 1) for p in blas] or [1])
    t = workload_tensors(w, with_dout=with_bwd)
    scale = default_scale(w.d)
    per_head = fwd_flop(1, 1, w.N, w.d, causal) * (3.5 if with_bwd else 1.0)
    heads = 0
    start = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            q, k, v = (bf16_bits_to_f64(t[x][sl]) for x in ("q", "k", "v"))
            attention_forward(q, k, v, causal=causal, scale=scale)
            if with_bwd:
                attention_backward(q, k, v, bf16_bits_to_f64(t["dout"][sl]), causal=causal,
                                   scale=scale)
            heads += 1
            if time.perf_counter() - start >= budget_s:
                break
        if time.perf_counter() - start >= budget_s:
            break
    el = time.perf_counter() - start
    return {
        "value": per_head * heads / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.H} (batch, head) slices, "
                   f"{'forward+backward' if with_bwd else 'forward'}, float64 numpy, "
                   f"{el:.1f} s"),
        "cpu_model": cpu_model(),
        "logical_cpus": os.cpu_count(),
        "blas": ", ".join(f"{p.get('internal_api')} {p.get('version')} "
                          f"({p.get('threading_layer')}, {p.get('num_threads')} threads)"
                          for p in blas) or "none found",
    }


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


FWD_SWEEP = ((2, False), (2, True), (3, True), (4, True), (4, False), (6, True), (6, False))


def forward_sweep(fa2, torch, dev, reps=10, warm_ms=60.0):
    """Forward-only TFLOP/s of the forward workloads (B=8 H=32 N=2048 d=64 both masks,
    B=4 H=16 N=4096 d=128 causal, B=1 H=16 N=16384 d=128 both masks, B=2 H=16 N=4096 d=256
    both masks). All inputs are made
    and copied to the device first; each case then runs back to back for at least `warm_ms`
    of GPU time before `reps` calls are timed with HIP events on the launch stream."""
    import numpy as np

    from exact_io_aware_42_amd.inputs import WORKLOADS, default_scale, workload_tensors

    stream = torch.cuda.current_stream(dev)
    dev_inputs = {}
    for wid in sorted({wid for wid, _ in FWD_SWEEP}):
        t = workload_tensors(WORKLOADS[wid])
        dev_inputs[wid] = [torch.from_numpy(t[x].view(np.int16)).view(torch.bfloat16).to(dev)
                           for x in ("q", "k", "v")]
    torch.cuda.synchronize()
    res = {}
    for wid, causal in FWD_SWEEP:
        w = WORKLOADS[wid]
        q, k, v = dev_inputs[wid]
        o = torch.empty_like(q)
        lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
        run = lambda: fa2.fwd(q, k, v, causal=causal, scale=default_scale(w.d), out=o, lse=lse)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        for _ in range(max(2, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
            run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for r in range(reps):
            run()
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        ms = sum(ev[r].elapsed_time(ev[r + 1]) for r in range(reps)) / reps
        tf = fwd_flop(*w.shape, causal) / (ms * 1e-3) / 1e12
        res[f"{w.name} {'causal' if causal else 'non-causal'}"] = {
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return res


def gpt_layer_step(torch, dev, steps=20, warmup=10):
    """Forward+backward of a GPT-style causal attention layer (bf16 QKV and output projections
    by torch matmul, attention by flash_attn_func) at the GPT-style workload's shape
    (B=4, N=4096, H=16, d=128, C=2048), synthetic weights and data."""
    from exact_io_aware_42_amd.gpt_layer import layer_flop, layer_forward, make_params

    B, N, H, d = 4, 4096, 16, 128
    x, w_qkv, w_o, dy = make_params(B, N, H, d, dev, seed=7)

    def step():
        for t in (x, w_qkv, w_o):
            t.grad = None
        layer_forward(x, w_qkv, w_o, H).backward(dy)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = layer_flop(B, N, H, d)
    total = fl["projections"] + fl["attention"]
    return {"shape": f"B{B} N{N} H{H} d{d} C{H * d} causal", "ms_per_step": round(ms, 4),
            "tflops": round(total / (ms * 1e-3) / 1e12, 1),
            "attention_flop_share": round(fl["attention"] / total, 3)}


def _timed_fwd_bwd(fa2, torch, dev, H, Hkv, steps, warmup, warm_ms=WARM_MS, **kw):
    """Mean time (ms) of fwd + bwd at B=4, N=2048, d=128, causal, with H query heads and Hkv K/V
    heads; i.i.d. N(0,1) bf16 from a seeded torch generator. kw goes to fwd and bwd. As for the
    main step: outputs and workspace given by the caller (the workspace sized for the split of
    small problems), at least warm_ms of GPU time untimed, then `warmup` untimed steps."""
    B, N, d = 4, 2048, 128
    g = torch.Generator(device="cpu").manual_seed(11)
    mk = lambda h: torch.randn(B, h, N, d, generator=g).to(torch.bfloat16).to(dev)
    q, k, v, do = mk(H), mk(Hkv), mk(Hkv), mk(H)
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, fa2.bwd_workspace_bytes(B, H, N, d, Hkv)), dtype=torch.uint8,
                     device=dev)

    def step():
        fa2.fwd(q, k, v, causal=True, out=o, lse=lse, **kw)
        fa2.bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spent = 0.0
    while spent < warm_ms:
        e0.record()
        for _ in range(10):
            step()
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 3.5 * fwd_flop(B, H, N, d, True)
    return {"ms_per_step": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}


def gqa_step(fa2, torch, dev, steps=20, warmup=20):
    """Forward+backward with grouped K/V heads at the fwd+bwd workload's shape: B=4, H=16
    query heads sharing Hkv=4 K/V heads (groups of 4), N=2048, d=128, causal. FLOP as for 16
    full heads."""
    r = _timed_fwd_bwd(fa2, torch, dev, 16, 4, steps, warmup)
    return {"shape": "B4 H16 Hkv4 N2048 d128 causal", **r}


def dropout_step(fa2, torch, dev, p=0.1, steps=20, warmup=20):
    """Forward+backward with dropout p on the attention probabilities (mask regenerated from
    the counter-based hash in every kernel) at the fwd+bwd workload's shape: B=4, H=16,
    N=2048, d=128, causal. FLOP as without dropout (the hash work is not counted)."""
    r = _timed_fwd_bwd(fa2, torch, dev, 16, 16, steps, warmup, dropout_p=p, seed=1234,
                       offset=0)
    return {"shape": "B4 H16 N2048 d128 causal", "dropout_p": p, **r}


def gemm_yardstick(torch, dev, n=8192, steps=20, warm_ms=WARM_MS):
    """A library bf16 GEMM on the same chip, for context: C = A B with A, B [n, n] bf16 (fp32
    accumulation) through torch.matmul (the ROCm BLAS libraries), after warm_ms of untimed GEMMs.
    2 n^3 FLOP each. Not part of `value`."""
    g = torch.Generator(device="cpu").manual_seed(17)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spent = 0.0
    while spent < warm_ms:
        e0.record()
        for _ in range(5):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
    e0.record()
    for _ in range(steps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": f"{n}x{n}x{n} bf16, torch.matmul", "ms": round(ms, 4),
            "tflops": round(tflops, 1), "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}


def graph_step(fa2, torch, dev, steps=100, warmup=20, warm_ms=WARM_MS):
    """The fwd+bwd step at the default workload's shape (B=4, H=16, N=2048, d=128, causal) with
    caller-given outputs and workspace, captured once in a HIP graph and replayed: the launch
    overhead floor of the step. Reported beside the same calls made eagerly on the same
    inputs; not part of `value`."""
    B, H, N, d = 4, 16, 2048, 128
    g = torch.Generator(device="cpu").manual_seed(13)
    mk = lambda: torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    q, k, v, do = mk(), mk(), mk(), mk()
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def step():
        fa2.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa2.bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(run):
        # at least warm_ms of GPU time untimed (as for the main step), then `warmup` more runs
        spent = 0.0
        while spent < warm_ms:
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                run()
            e1.record()
            torch.cuda.synchronize()
            spent += e0.elapsed_time(e1)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    eager_ms = timed(step)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_ms = timed(graph.replay)
    flop = 3.5 * fwd_flop(B, H, N, d, True)
    return {"shape": "B4 H16 N2048 d128 causal", "ms_per_step": round(graph_ms, 4),
            "tflops": round(flop / (graph_ms * 1e-3) / 1e12, 1),
            "eager_ms_per_step": round(eager_ms, 4)}


def measure_step(fa2, torch, dev, w, causal, with_bwd, steps, warmup, warm_ms=WARM_MS):
    """Run untimed steps (forward, then dQ and dK/dV) of workload `w` for at least `warm_ms` of
    GPU time (the clock needs a few hundred milliseconds of load to settle; a step count alone
    left short runs about 10% low), then `warmup` more untimed steps and `steps` timed ones.
    Inside the timed steps only the last stage (dK/dV, or the forward alone) is bracketed by
    HIP events on the launch stream: each event record costs the step about 2 us. The other
    stages are timed the same way over a further min(steps, 20) steps after the timed region.
    Returns (stage names, their algorithmic FLOP, step FLOP, mean stage ms, wall seconds of the
    timed steps, GPU milliseconds of the time-based warm-up)."""
    import numpy as np

    from exact_io_aware_42_amd.inputs import default_scale, workload_tensors

    B, H, N, d = w.shape
    scale = default_scale(d)
    t = workload_tensors(w, with_dout=with_bwd)

    def dev_t(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_t(t["q"]), dev_t(t["k"]), dev_t(t["v"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if with_bwd:
        do = dev_t(t["dout"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(1, fa2.bwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8,
                         device=dev)

    stream = torch.cuda.current_stream(dev)
    kernels = ["fa2_fwd_kernel"]
    if with_bwd:
        # dK/dV without dropout runs fa2_bwd_dkdv16_kernel at every head dimension
        kernels += ["fa2_bwd_dq_kernel", "fa2_bwd_dkdv16_kernel"]
    f_fwd = fwd_flop(B, H, N, d, causal)
    algo_flop = {"fa2_fwd_kernel": f_fwd, "fa2_bwd_dkdv16_kernel": 2.0 * f_fwd,
                 "fa2_bwd_dq_kernel": 0.5 * f_fwd}
    step_flop = f_fwd * (3.5 if with_bwd else 1.0)

    def step(events=None, marks=()):
        def mark(i):
            if events is not None and i in marks:
                events[i].record(stream)
        mark(0)
        fa2.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        mark(1)
        if with_bwd:
            # dQ first: it also stores D = rowsum(dO * O) and LSE*log2(e) for dK/dV
            fa2.bwd_dq(q, k, v, o, do, lse, ws, causal=causal, scale=scale, dq=dq)
            mark(2)
            fa2.bwd_dkdv(q, k, v, do, ws, causal=causal, scale=scale, dk=dk, dv=dv)
            mark(3)

    # time-based warm-up: batches of steps until warm_ms of GPU time have passed
    warm_done = 0.0
    batch = 1
    while warm_done < warm_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            step()
        e1.record(stream)
        e1.synchronize()
        warm_done += e0.elapsed_time(e1)
        batch = min(batch * 2, 256)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    n_ev = len(kernels) + 1
    last = (n_ev - 2, n_ev - 1)  # the events around the last stage
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i], last)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def mean_ms(evs, i):
        durs = [e[i].elapsed_time(e[i + 1]) for e in evs]
        return sum(durs) / len(durs)

    kernel_ms = {kernels[-1]: mean_ms(ev, n_ev - 2)}
    if len(kernels) > 1:
        n2 = min(steps, 20)
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n2)]
        for i in range(n2):
            step(ev2[i], tuple(range(n_ev)))
        torch.cuda.synchronize()
        for i, kname in enumerate(kernels[:-1]):
            kernel_ms[kname] = mean_ms(ev2, i)
    return kernels, algo_flop, step_flop, kernel_ms, elapsed, warm_done


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1 "
                          "(the per-head work is independent, so more GPUs would shard "
                          "batch x heads without any exchange)"}))
        sys.exit(2)

    import torch

    import exact_io_aware_42_amd as fa2
    from exact_io_aware_42_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    causal = w.causal_modes[0] if args.causal == "default" else args.causal == "causal"
    with_bwd = args.direction == "both"
    B, H, N, d = w.shape
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa2.load_library()

    kernels, algo_flop, step_flop, kernel_ms, elapsed, warm_done = measure_step(
        fa2, torch, dev, w, causal, with_bwd, args.steps, args.warmup)
    ms_per_step = elapsed * 1e3 / args.steps

    # the roofline kernel is the last stage, the one timed inside the timed steps: dK/dV for the
    # fwd+bwd step (its largest time share), the forward alone otherwise
    dominant = kernels[-1]
    achieved = algo_flop[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12
    wtag = f"w{w.wid}_{'causal' if causal else 'full'}"
    from exact_io_aware_42_amd.profiling import load_traffic
    traffic = load_traffic(dominant, wtag)

    value = step_flop * args.steps / elapsed / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_gpu_ms": round(warm_done, 1),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) rounded to bf16, seeded (seed = 1000*workload + t)",
        "config": {
            "workload": w.name,
            "B": B, "H": H, "N": N, "d": d,
            "causal": causal,
            "direction": "fwd+bwd" if with_bwd else "fwd",
            "step_flop": step_flop,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernel_ms": {kn: round(v_, 5) for kn, v_ in kernel_ms.items()},
        "kernel_tflops": {kn: (round(algo_flop[kn] / (kernel_ms[kn] * 1e-3) / 1e12, 2)
                               if algo_flop[kn] else None) for kn in kernels},
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_fwd_sweep:
        out["forward_workloads"] = forward_sweep(fa2, torch, dev)
        if args.workload == 5 and with_bwd and causal:
            # before the GEMM-heavy layer step, each side after its own time-based warm-up
            out["graph_step"] = graph_step(fa2, torch, dev)

        def other_step(wo, co):
            kn, af, sf, km, el, _ = measure_step(fa2, torch, dev, wo, co, True, 20, 20)
            return {"ms_per_step": round(el * 1e3 / 20, 4),
                    "tflops": round(sf * 20 / el / 1e12, 1),
                    "kernel_ms": {k_: round(v_, 4) for k_, v_ in km.items()},
                    "kernel_tflops": {k_: round(af[k_] / (km[k_] * 1e-3) / 1e12, 1) for k_ in kn}}

        # the same fwd+bwd step without the causal mask (the metric names both masks), and the
        # fwd+bwd step at head dimension 256 (both masks)
        if w.backward and causal:
            out["non_causal_step"] = {f"{w.name} non-causal fwd+bwd": other_step(w, False)}
        w6 = WORKLOADS[6]
        out["d256_steps"] = {f"{w6.name} {'causal' if c6 else 'non-causal'} fwd+bwd":
                             other_step(w6, c6) for c6 in (True, False)}
        out["gpt_layer_step"] = gpt_layer_step(torch, dev)
        out["gqa_step"] = gqa_step(fa2, torch, dev)
        out["dropout_step"] = dropout_step(fa2, torch, dev)
        out["gemm_yardstick"] = gemm_yardstick(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, causal, with_bwd, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
