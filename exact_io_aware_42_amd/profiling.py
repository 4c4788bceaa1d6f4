"""HBM-traffic accounting from rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE).

    # a plain device copy of known size, to calibrate the counters
    python -m exact_io_aware_42_amd.profiling copy --mib 256
    # turn a rocprofv3 --stats kernel_stats.csv into a short text summary
    python -m exact_io_aware_42_amd.profiling stats --csv run_kernel_stats.csv \
        --out profiles/kernels_<workload>.txt --title "..." --cmd "rocprofv3 ..."
    # the same from run_kernel_trace.csv, one line per (kernel, grid size); --last N keeps
    # the last N dispatches of each line (the timed steps after the warm-up); --workgroups
    # keeps only launches of the given grid sizes; --stop-at 'kernel|workgroups' adds a table
    # of the dispatches before that launch (a benchmark's main loop, before its other cases)
    python -m exact_io_aware_42_amd.profiling trace --csv run_kernel_trace.csv \
        --out profiles/kernels_<workload>.txt --title "..." --cmd "rocprofv3 ..." [--last N]
    # effective clock per kernel: GRBM_GUI_ACTIVE (summed over the 8 XCDs) of each dispatch
    # over its kernel-trace duration, from one rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE run
    python -m exact_io_aware_42_amd.profiling clock --dir <rocprofv3 output dir> \
        --out profiles/clock_<workload>.txt --title "..." --cmd "rocprofv3 ..."
    # SQ counter summary per kernel (median per dispatch over one or more --pmc passes, each
    # pass its own counter_collection.csv) with the derived busy fractions
    python -m exact_io_aware_42_amd.profiling counters --csv pass1.csv pass2.csv ... \
        --out profiles/counters_<workload>.txt --title "..." --cmd "rocprofv3 ..."
    # turn counter CSVs into profiles/traffic_<kernel>_<workload>.txt
    python -m exact_io_aware_42_amd.profiling traffic --kernel fa2_fwd_kernel \\
        --workload w4_full --fetch run_fetch.csv --write run_write.csv \\
        --copy-fetch copy_fetch.csv --copy-write copy_write.csv --copy-mib 256

The counters report KiB per dispatch; the copy of known size gives the factor between what a
counter reads and the bytes that actually moved (fetch: bytes read, write: bytes written).
The summary records a digest of the kernel's sources so that a stale summary is not used.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)

KERNEL_SOURCES = {
    "fa2_fwd_kernel": ["fa2_device.hpp", "fa2_fwd.hip"],
    "fa2_bwd_dkdv16_kernel": ["fa2_device.hpp", "fa2_bwd.hip"],
    "fa2_bwd_dq_kernel": ["fa2_device.hpp", "fa2_bwd.hip"],
    "fa2_bwd_pre_kernel": ["fa2_device.hpp", "fa2_bwd.hip"],
}


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one space (string
    literals are kept as they are; the kernel sources hold none with comment markers)."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest(kernel: str) -> str:
    """Digest of the code (comments and layout excluded) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG_DIR, "csrc", n)) as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_path(kernel: str, workload_tag: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_tag}.txt")


def load_traffic(kernel: str, workload_tag: str):
    """HBM bytes per launch from a committed summary, or None if absent or stale."""
    path = traffic_path(kernel, workload_tag)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_source_digest(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counter_values(path: str, counter: str, name_substr: str):
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {name_substr!r} in {path}")
    return vals


def copy_main(mib: int):
    import torch

    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB three times", flush=True)


def short_name(name: str) -> str:
    """'void fa2::(anonymous namespace)::fa2_fwd_kernel<128, true>(...)' -> 'fa2_fwd_kernel<128,
    true>'."""
    head = name.split("(", 1)[0] if "(anonymous" not in name else name
    head = head.replace("void ", "").replace("fa2::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in head:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def stats_main(a):
    rows = []
    with open(a.csv) as f:
        for r in csv.DictReader(f):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    with open(a.out, "w") as f:
        f.write(f"# rocprofv3 kernel statistics: {a.title}\n")
        f.write(f"# command: {a.cmd}\n")
        f.write("# kernel | calls | average us | min us | max us | share of GPU time\n")
        for n, c, avg, mn, mx, pct in rows:
            f.write(f"{n} | {c} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}%\n")
    print(open(a.out).read())


def trace_main(a):
    groups = {}
    with open(a.csv) as f:
        for r in csv.DictReader(f):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
            if a.workgroups and key[1] not in a.workgroups:
                continue
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append((int(r["Start_Timestamp"]), dur))
    for v in groups.values():
        v.sort()
    total = sum(d for v in groups.values() for _, d in v)

    def table(sel_groups):
        rows = []
        for (name, wgs), v in sel_groups.items():
            if not v:
                continue
            sel = [d for _, d in v][-a.last:] if a.last else [d for _, d in v]
            rows.append((name, wgs, len(v), len(sel), statistics.mean(sel), min(sel), max(sel),
                         100.0 * sum(d for _, d in v) / total))
        rows.sort(key=lambda x: -x[7])
        return rows

    with open(a.out, "w") as f:
        f.write(f"# rocprofv3 kernel trace: {a.title}\n")
        f.write(f"# command: {a.cmd}\n")
        head = ("# kernel | workgroups | dispatches | dispatches averaged (last) | average us | "
                "min us | max us | share of GPU time\n")
        if a.stop_at:
            # the leading segment: every dispatch before the first launch of the given
            # (kernel, workgroup count), e.g. the first kernel after a benchmark's main loop
            name, wgs = a.stop_at.rsplit("|", 1)
            stops = [t for (n, w), v in groups.items() if n == name and w == int(wgs) for t, _ in v]
            if not stops:
                raise SystemExit(f"no launch of {a.stop_at!r} in {a.csv}")
            t_stop = min(stops)
            lead = {k: [x for x in v if x[0] < t_stop] for k, v in groups.items()}
            f.write(f"# segment before the first launch of {name} on {wgs} workgroups; the last "
                    f"{a.last} dispatches of each line in it are averaged\n")
            f.write(head)
            for n, w, c, k, avg, mn, mx, pct in table(lead):
                f.write(f"{n} | {w} | {c} | {k} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}%\n")
            f.write("# the whole run\n")
        f.write(head)
        for n, w, c, k, avg, mn, mx, pct in table(groups):
            f.write(f"{n} | {w} | {c} | {k} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}%\n")
    print(open(a.out).read())


def clock_main(a):
    counters, names, durs = {}, {}, {}
    with open(os.path.join(a.dir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                did = int(r["Dispatch_Id"])
                counters[did] = float(r["Counter_Value"])
                names[did] = short_name(r["Kernel_Name"])
    with open(os.path.join(a.dir, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            durs[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
    groups = {}
    for did, c in counters.items():
        if did in durs:
            groups.setdefault(names[did], []).append((did, c, durs[did]))
    with open(a.out, "w") as f:
        f.write(f"# effective shader clock: {a.title}\n")
        f.write(f"# command: {a.cmd}\n")
        f.write("# GRBM_GUI_ACTIVE per dispatch is summed over the 8 XCDs; clock = value / 8 / "
                "duration. Second half of the dispatches (after warm-up).\n")
        f.write("# kernel | dispatches used | average us | GRBM_GUI_ACTIVE / 8 | clock GHz\n")
        for n, v in sorted(groups.items()):
            v.sort()
            v = v[len(v) // 2:]
            c = statistics.mean(x[1] for x in v) / 8
            t = statistics.mean(x[2] for x in v)
            f.write(f"{n} | {len(v)} | {t * 1e6:.1f} | {c:.4g} | {c / t / 1e9:.3f}\n")
    print(open(a.out).read())


# gfx950 part: 8 XCDs of 32 CUs, 4 SIMDs per CU; GRBM_GUI_ACTIVE is summed over the XCDs,
# SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs (32 per 32x32x16 MFMA), SQ_LDS_IDX_ACTIVE over the
# CUs, SQ_WAVE_CYCLES and the SQ_WAIT_* / SQ_ACTIVE_INST_* counters over the waves.
XCDS, CUS, SIMDS_PER_CU = 8, 256, 4


def counters_main(a):
    vals = {}
    for path in a.csv:
        with open(path) as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    with open(a.out, "w") as f:
        f.write(f"# SQ counters per dispatch (median): {a.title}\n")
        f.write(f"# command: {a.cmd}\n")
        f.write("# derived: kernel cycles = GRBM_GUI_ACTIVE / 8 (per XCD); MFMA busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles * 1024 SIMDs); LDS active = "
                "SQ_LDS_IDX_ACTIVE / (kernel cycles * 256 CUs); wait/active shares are of "
                "SQ_WAVE_CYCLES\n")
        for k in sorted(vals):
            m = {c: statistics.median(v) for c, v in vals[k].items()}
            f.write(f"{k}\n")
            for c in sorted(m):
                f.write(f"    {c:28s} {m[c]:.6g}\n")
            cyc = m.get("GRBM_GUI_ACTIVE", 0) / XCDS
            if cyc:
                if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                    f.write(f"    -> MFMA busy {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * CUS * SIMDS_PER_CU):.3f}\n")
                if "SQ_LDS_IDX_ACTIVE" in m:
                    f.write(f"    -> LDS active {m['SQ_LDS_IDX_ACTIVE'] / (cyc * CUS):.3f}\n")
            wc = m.get("SQ_WAVE_CYCLES")
            if wc:
                for c in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                          "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
                    if c in m:
                        f.write(f"    -> {c} / SQ_WAVE_CYCLES {m[c] / wc:.3f}\n")
            if m.get("SQ_INSTS_MFMA"):
                for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                    if c in m:
                        f.write(f"    -> {c} per MFMA {m[c] / m['SQ_INSTS_MFMA']:.2f}\n")
    print(open(a.out).read())


def traffic_main(a):
    fetch = statistics.median(counter_values(a.fetch, "FETCH_SIZE", a.kernel))
    write = statistics.median(counter_values(a.write, "WRITE_SIZE", a.kernel))
    # the copy kernel is the only kernel in the calibration runs besides the fill
    copy_bytes = a.copy_mib * 1024 * 1024
    cf = counter_values(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = counter_values(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_fetch = copy_bytes / (statistics.median(cf) * 1024)
    f_write = copy_bytes / (statistics.median(cw) * 1024)
    traffic = fetch * 1024 * f_fetch + write * 1024 * f_write
    out = traffic_path(a.kernel, a.workload)
    with open(out, "w") as f:
        f.write(f"# HBM traffic of {a.kernel} on workload {a.workload}, from rocprofv3 counters\n")
        f.write(f"# command (fetch pass): {a.cmd_fetch}\n")
        f.write(f"# command (write pass): {a.cmd_write}\n")
        f.write(f"# calibration: {a.copy_mib} MiB device copy (torch copy_), "
                f"kernel matching {a.copy_kernel!r}\n")
        f.write(f"kernel_source_digest: {kernel_source_digest(a.kernel)}\n")
        f.write(f"fetch_kib_per_dispatch: {fetch:.1f}\n")
        f.write(f"write_kib_per_dispatch: {write:.1f}\n")
        f.write(f"copy_fetch_factor: {f_fetch:.4f}\n")
        f.write(f"copy_write_factor: {f_write:.4f}\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
    print(open(out).read())


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="sub", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=256)
    st = sub.add_parser("stats")
    st.add_argument("--csv", required=True)
    st.add_argument("--out", required=True)
    st.add_argument("--title", required=True)
    st.add_argument("--cmd", required=True)
    tr = sub.add_parser("trace")
    tr.add_argument("--csv", required=True)
    tr.add_argument("--out", required=True)
    tr.add_argument("--title", required=True)
    tr.add_argument("--cmd", required=True)
    tr.add_argument("--last", type=int, default=0)
    tr.add_argument("--workgroups", type=lambda x: [int(v) for v in x.split(",")], default=None,
                    help="keep only launches with these workgroup counts")
    tr.add_argument("--stop-at", default=None,
                    help="'kernel|workgroups': also summarise the dispatches before its first launch")
    ck = sub.add_parser("clock")
    ck.add_argument("--dir", required=True)
    ck.add_argument("--out", required=True)
    ck.add_argument("--title", required=True)
    ck.add_argument("--cmd", required=True)
    cn = sub.add_parser("counters")
    cn.add_argument("--csv", required=True, nargs="+")
    cn.add_argument("--out", required=True)
    cn.add_argument("--title", required=True)
    cn.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, default=256)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--cmd-fetch", default="")
    t.add_argument("--cmd-write", default="")
    a = ap.parse_args(argv)
    if a.sub == "copy":
        copy_main(a.mib)
    elif a.sub == "stats":
        stats_main(a)
    elif a.sub == "trace":
        trace_main(a)
    elif a.sub == "clock":
        clock_main(a)
    elif a.sub == "counters":
        counters_main(a)
    else:
        traffic_main(a)


if __name__ == "__main__":
    main(sys.argv[1:])
