"""Turn rocprofv3 CSV output of bench.py runs into the text summaries kept
under profiles/.

    python profile_summary.py kernels  OUT.md KT_DIR  [--command CMD] [--skip N]
    python profile_summary.py traffic  OUT.md FETCH_CSV WRITE_CSV CAL_FETCH_CSV CAL_WRITE_CSV
                                       [--workload NAME] [--command CMD ...]
    python profile_summary.py syncs    OUT.md TRACE_DIR [--command CMD]
    python profile_summary.py mfma     OUT.md COUNTER_CSV [--workload NAME] [--command CMD]

`kernels` summarises a `--kernel-trace --stats` run (the *_kernel_stats.csv
file in KT_DIR). `traffic` takes one `--pmc FETCH_SIZE` and one
`--pmc WRITE_SIZE` run of the same bench command, plus the same two counters
over `bench.py --copy-calibration MIB` (plain copies of a known size), and
writes per-stage HBM bytes per launch: each counter is scaled by
(bytes the copy moves) / (what the counter reads for it). The traffic file
ends with a JSON block that bench.py reads for `roofline.traffic`; each entry
carries the hash of the kernel sources it was measured on, so a later kernel
change turns the figure back into null.

`syncs` reads a `--kernel-trace --memory-copy-trace --hip-runtime-trace` run
and checks each layer step, from the host call that launches its first
kernel to the one that launches its last, for HIP calls that block the host,
copy memory or allocate, and the GPU span of each step for device-to-host
copies.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

GG_OPS = ["gg_fwd_gate_up", "gg_fwd_down", "gg_dgrad_down", "gg_dgrad_gate_up",
          "gg_wgrad_down", "gg_wgrad_gate_up"]
ROW_KERNELS = [
    ("combine_bwd_kernel", "combine_bwd"), ("combine_bwd_rows_kernel", "combine_bwd"),
    ("permute_bwd_kernel", "permute_bwd"),
    ("combine_kernel", "combine"), ("permute_kernel", "permute"),
    ("zero_pad_rows_kernel", "permute"),
    ("hist_kernel", "offsets"), ("scan_kernel", "offsets"), ("rank_kernel", "offsets"),
    ("router_gemm_kernel", "router_gemm"), ("router_gemm_lds_kernel", "router_gemm"),
    ("router_gemm_mfma_kernel", "router_gemm"), ("router_bwd_mfma_kernel", "router_gemm_bwd"),
    ("route_bwd_kernel", "route_bwd"), ("route_kernel", "route"),
    ("router_bwd_partial_kernel", "router_gemm_bwd"), ("router_bwd_reduce_kernel", "router_gemm_bwd"),
]
TRAFFIC_BEGIN = "<!-- traffic-json -->"


def stage_of(kernel):
    """Pipeline stage a kernel belongs to, or None for library kernels."""
    m = re.search(r"moe::gg_mx(?:_wgrad_split)?_kernel<(\d+),", kernel)
    if m:
        return "mx" + GG_OPS[int(m.group(1))][2:]
    m = re.search(r"moe::gg_\w+_kernel<(\d+)[,>]", kernel)
    if m:
        return GG_OPS[int(m.group(1))]
    if re.search(r"moe::(\(anonymous namespace\)::)?mx_(both|rows|cols)_kernel", kernel):
        return "mx_quantize"
    for pat, st in ROW_KERNELS:
        if re.search(r"moe::" + pat + r"\b", kernel):
            return st
    return None


def short(kernel):
    m = re.search(r"moe::(\w+)(<[^()]*>)?", kernel)
    if not m:
        return kernel[:60]
    return m.group(1) + (m.group(2) or "")


def _timed_means(trace_path, skip):
    """Mean duration (us) of each kernel over its launches after the first
    `skip` (the warm-up steps of the traced bench run), in launch order."""
    runs = {}
    for r in csv.DictReader(open(trace_path)):
        runs.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, v in runs.items():
        v.sort()
        kept = [ns for _, ns in v[skip:]] or [ns for _, ns in v]
        out[name] = sum(kept) / len(kept) / 1e3
    return out


def kernels(args):
    path = glob.glob(os.path.join(args.dir, "*kernel_stats.csv"))
    if len(path) != 1:
        sys.exit(f"expected one *kernel_stats.csv under {args.dir}, found {path}")
    rows = list(csv.DictReader(open(path[0])))
    trace = glob.glob(os.path.join(args.dir, "*kernel_trace.csv"))
    timed = _timed_means(trace[0], args.skip) if len(trace) == 1 else {}
    out = ["# Kernel durations", ""]
    if args.command:
        out += ["Command (from the repository root):", "", "```", args.command, "```", ""]
    out += ["Source: rocprofv3 `--kernel-trace --stats` (kernel_stats.csv, kernel_trace.csv). "
            "`avg us` includes the warm-up launches; `timed avg us` leaves out each kernel's "
            f"first {args.skip} launches (the bench's warm-up steps), which is what bench.py "
            "times.", "",
            "| stage | kernel | calls | avg us | timed avg us | min us | max us | % of GPU time |",
            "|---|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        t = timed.get(r["Name"])
        out.append("| {} | `{}` | {} | {:.1f} | {} | {:.1f} | {:.1f} | {:.2f} |".format(
            stage_of(r["Name"]) or "-", short(r["Name"]), r["Calls"],
            float(r["AverageNs"]) / 1e3, "-" if t is None else f"{t:.1f}",
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    open(args.out, "w").write("\n".join(out) + "\n")
    print(args.out)


def _counter(path, name):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == name]
    if not rows:
        sys.exit(f"no {name} rows in {path}")
    return rows


def _calibration(path, name, copy_bytes):
    """Counter KiB reported for the plain copies -> bytes per counted KiB."""
    rows = [r for r in _counter(path, name) if "copyBuffer" in r["Kernel_Name"]]
    if not rows:
        sys.exit(f"no copy kernels in {path}")
    kib = sum(float(r["Counter_Value"]) for r in rows) / len(rows)
    direction = copy_bytes  # a copy reads and writes copy_bytes each
    return direction / kib, kib


def _per_stage(path, name):
    """Mean counter KiB per launch of each stage (kernels of one stage summed
    within a step: a stage's kernels run once per step)."""
    tot, calls = {}, {}
    for r in _counter(path, name):
        st = stage_of(r["Kernel_Name"])
        if st is None:
            continue
        tot[st] = tot.get(st, 0.0) + float(r["Counter_Value"])
        k = short(r["Kernel_Name"])
        calls.setdefault(st, {}).setdefault(k, 0)
        calls[st][k] += 1
    return {st: tot[st] / max(calls[st].values()) for st in tot}


def traffic(args):
    from bench import kernel_source_hash, stage_algorithmic_bytes
    from moe_inputs import workload
    wl = workload(args.workload)
    copy_bytes = args.copy_mib * (1 << 20)
    f_scale, f_kib = _calibration(args.cal_fetch, "FETCH_SIZE", copy_bytes)
    w_scale, w_kib = _calibration(args.cal_write, "WRITE_SIZE", copy_bytes)
    fetch = _per_stage(args.fetch, "FETCH_SIZE")
    write = _per_stage(args.write, "WRITE_SIZE")
    h = kernel_source_hash()
    out = ["# HBM traffic per launch: " + args.workload, ""]
    if args.command:
        out += ["Commands (from the repository root):", "", "```"] + args.command + ["```", ""]
    out += [f"Calibration: a plain copy of {args.copy_mib} MiB reads {f_kib:.0f} KiB on "
            f"FETCH_SIZE and writes {w_kib:.0f} KiB on WRITE_SIZE, so FETCH_SIZE is scaled by "
            f"{f_scale / 1024:.3f} and WRITE_SIZE by {w_scale / 1024:.3f} (bytes per counted "
            "byte). FETCH_SIZE counts L2 misses, some of which the MALL may serve.", "",
            f"Kernel sources hash: `{h}`", "",
            "| stage | FETCH KiB | WRITE KiB | traffic MB | algorithmic MB | traffic / algorithmic |",
            "|---|---:|---:|---:|---:|---:|"]
    tab = {}
    R = wl.T * wl.k
    for st in sorted(fetch, key=lambda s: -(fetch[s] * f_scale + write.get(s, 0) * w_scale)):
        b = fetch[st] * f_scale + write.get(st, 0.0) * w_scale
        alg = stage_algorithmic_bytes(st, wl, R, R)
        out.append("| {} | {:.0f} | {:.0f} | {:.1f} | {:.1f} | {:.2f} |".format(
            st, fetch[st], write.get(st, 0.0), b / 1e6, alg / 1e6, b / alg))
        tab[st] = {"bytes_per_launch": round(b), "source_hash": h}
    out += ["", TRAFFIC_BEGIN, "```json", json.dumps({args.workload: tab}, indent=1), "```"]
    open(args.out, "w").write("\n".join(out) + "\n")
    print(args.out)


def read_traffic_table(path):
    """The JSON block of a traffic summary (bench.py reads it)."""
    txt = open(path).read()
    i = txt.find(TRAFFIC_BEGIN)
    if i < 0:
        return {}
    body = txt[i:].split("```json", 1)[1].split("```", 1)[0]
    return json.loads(body)


def mfma(args):
    """Matrix-core busy fraction (rocprofv3's MfmaUtil: MFMA busy cycles over
    active cycles x SIMDs) and executed bf16 MFMA work (SQ_INSTS_VALU_MFMA_MOPS_BF16
    x 512 flops) per grouped-GEMM launch, against the algorithmic flops."""
    from bench import stage_work
    from moe_inputs import workload
    wl = workload(args.workload)
    R = wl.T * wl.k
    skip = getattr(args, "skip", 0)
    vals = {}
    for r in csv.DictReader(open(args.csv)):
        st = stage_of(r["Kernel_Name"])
        if st is None or not st.startswith("gg_") or "split_kernel" in r["Kernel_Name"]:
            continue
        vals.setdefault(st, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["# Matrix-core utilisation of the grouped GEMMs: " + wl.name, ""]
    if args.command:
        out += ["Command (from the repository root):", "", "```", args.command, "```", ""]
    span = (f"launches after each kernel's first {skip} (the bench's warm-up steps)" if skip
            else "launches")
    out += ["Source: rocprofv3 `--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16`, means over the run's "
            f"{span}. `MfmaUtil` is the fraction of SIMD cycles with the matrix core busy while the GPU "
            "is active (so it is measured against the clock the GPU actually ran at); executed GFLOP "
            "counts every MFMA issued, including the zero rows of partial tiles.", "",
            "| stage | launches | MfmaUtil % | executed GFLOP | algorithmic GFLOP | executed / algorithmic |",
            "|---|---:|---:|---:|---:|---:|"]
    for st in GG_OPS:
        v = vals.get(st)
        if not v:
            continue
        util = v.get("MfmaUtil", [])[skip:]
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])[skip:]
        ex = sum(mops) / len(mops) * 512 / 1e9 if mops else float("nan")
        _, work = stage_work(st, wl, R, R)
        out.append(f"| {st} | {len(util)} | {sum(util) / max(len(util), 1):.1f} | {ex:.1f} | "
                   f"{work / 1e9:.1f} | {ex / (work / 1e9):.3f} |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print(args.out)


# HIP runtime calls that block the host, copy memory or allocate
HOST_BLOCKING = re.compile(r"^hip(DeviceSynchronize|StreamSynchronize|EventSynchronize|StreamWaitEvent|"
                           r"Memcpy\w*|Memset\w*|Malloc\w*|Free\w*|HostMalloc|HostRegister|"
                           r"MallocAsync|ModuleLoad\w*)$")


def syncs(args):
    one = lambda pat: (glob.glob(os.path.join(args.dir, pat)) or [None])[0]
    kt, api, cp = one("*kernel_trace.csv"), one("*hip_api_trace.csv"), one("*memory_copy_trace.csv")
    if kt is None or api is None:
        sys.exit(f"need *kernel_trace.csv and *hip_api_trace.csv under {args.dir}")
    calls = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Function"], int(r["Correlation_Id"]))
             for r in csv.DictReader(open(api))]
    by_corr = {c: (t0, t1) for t0, t1, _, c in calls}
    kern = []
    for r in csv.DictReader(open(kt)):
        st = stage_of(r["Kernel_Name"])
        if st is None:
            continue
        host = by_corr.get(int(r["Correlation_Id"]))
        kern.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), st, host))
    kern.sort()
    # a step starts at its first offsets kernel (after the router when routing is learned)
    first = "router_gemm" if any(k[2] == "router_gemm" for k in kern) else "offsets"
    steps, prev = [], None
    for k in kern:
        if k[2] == first and prev != first:
            steps.append([])
        if steps:
            steps[-1].append(k)
        prev = k[2]
    copies = []
    if cp is not None:
        copies = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Direction"])
                  for r in csv.DictReader(open(cp))]
    out = ["# Host synchronisation and copies inside the layer step", ""]
    if args.command:
        out += ["Command (from the repository root):", "", "```", args.command, "```", ""]
    out += ["Source: rocprofv3 kernel, memory-copy and HIP runtime traces. For each step: the host "
            "window from the call that launches the step's first kernel to the call that launches "
            "its last, the HIP runtime calls made in it, and the device-to-host copies that overlap "
            "the step's GPU span (its first kernel's start to its last kernel's end).", "",
            "| step | layer kernels | host window us | GPU span us | HIP calls in the window | "
            "blocking / copy / alloc calls | D2H copies |",
            "|---:|---:|---:|---:|---|---:|---:|"]
    bad_total = warm_bad = 0
    for i, st in enumerate(steps):
        hosts = [k[3] for k in st if k[3] is not None]
        h0, h1 = min(h[0] for h in hosts), max(h[1] for h in hosts)
        g0, g1 = st[0][0], max(k[1] for k in st)
        inside = [f for t0, t1, f, _ in calls if t0 >= h0 and t1 <= h1]
        hist = {}
        for f in inside:
            hist[f] = hist.get(f, 0) + 1
        bad = sum(n for f, n in hist.items() if HOST_BLOCKING.match(f))
        d2h = sum(1 for c0, c1, dr in copies if "DEVICE_TO_HOST" in dr and c1 >= g0 and c0 <= g1)
        if i < args.warmup:
            warm_bad += bad + d2h
        else:
            bad_total += bad + d2h
        desc = ", ".join(f"{f} {n}" for f, n in sorted(hist.items(), key=lambda x: -x[1]))
        tag = " (warm-up)" if i < args.warmup else ""
        out.append(f"| {i}{tag} | {len(st)} | {(h1 - h0) / 1e3:.1f} | {(g1 - g0) / 1e3:.1f} | {desc} | {bad} | {d2h} |")
    timed = max(len(steps) - args.warmup, 0)
    out += ["", f"Steps: {len(steps)}, of which the first {min(args.warmup, len(steps))} are the bench's warm-up: "
            "the layer allocates its activation and gradient buffers on first use, through torch's caching "
            f"allocator ({warm_bad} such calls there). Blocking, copying or allocating calls and device-to-host "
            f"copies inside the {timed} steps after the warm-up: {bad_total}."]
    open(args.out, "w").write("\n".join(out) + "\n")
    print(args.out)
    return bad_total


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("out")
    k.add_argument("dir")
    k.add_argument("--command")
    k.add_argument("--skip", type=int, default=2, help="warm-up launches per kernel to leave out")
    t = sub.add_parser("traffic")
    t.add_argument("out")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("cal_fetch")
    t.add_argument("cal_write")
    t.add_argument("--workload", default="e128_uniform_bf16")
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--command", action="append")
    y = sub.add_parser("syncs")
    y.add_argument("out")
    y.add_argument("dir")
    y.add_argument("--command")
    y.add_argument("--warmup", type=int, default=1, help="leading steps that are the bench's warm-up")
    m = sub.add_parser("mfma")
    m.add_argument("out")
    m.add_argument("csv")
    m.add_argument("--workload", default="e128_uniform_bf16")
    m.add_argument("--command")
    m.add_argument("--skip", type=int, default=0, help="warm-up launches per kernel to leave out")
    a = ap.parse_args()
    if a.mode == "mfma":
        return mfma(a)
    if a.mode == "syncs":
        sys.exit(1 if syncs(a) else 0)
    (kernels if a.mode == "kernels" else traffic)(a)


if __name__ == "__main__":
    main()
