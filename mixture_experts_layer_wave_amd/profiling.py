"""Summaries of rocprofv3 output for the layer's kernels (measurement tooling).

Two commands, both reading the CSV files that ``rocprofv3 --output-format csv`` writes:

``stats``   kernel-trace statistics (``*_kernel_stats.csv``) -> a Markdown table of every
            kernel's calls and average duration, plus per-stage sums (a stage is one call
            of the C ABI, e.g. the gated up-projection = its GEMM kernel + its split-K or
            stream-K fix-up kernel).
``mfma``    one counter run of the derived metrics MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over
            GRBM_GUI_ACTIVE x SIMDs) and MfmaFlopsBF16 (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512):
            per kernel with matrix-core work, the busy percentage and the bf16 flops it
            executed per dispatch, next to the useful flops of the stage when given.
``traffic`` two counter runs (``FETCH_SIZE`` and ``WRITE_SIZE``, KiB per dispatch) of the
            bench, and the same two counters for a device copy of known size whose reads
            use the GEMMs' direct-to-LDS copies. The copy gives the factor that turns
            counter KiB into bytes actually moved (bytes copied / counter bytes); the stage
            averages are scaled by it and written as JSON together with a hash of the
            kernel sources, so that a later change of the kernels invalidates them. The
            counters sit at the L2's memory-side interface: the bytes are L2 misses and
            write-backs, served by the Infinity Cache or by HBM (the counters cannot tell
            which).

Stage of a kernel: from its name and, for the templated GEMMs, the NB template argument
(2 = gated up-projection with two weight matrices, 1 = down-projection).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

STAGE_ORDER = ["route", "dispatch", "expert_up", "expert_down", "expert_ffn", "combine", "stats", "forward", "other"]


def _code_only(text: str) -> str:
    """Source text without comments and blank space (a comment edit changes no kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the kernel sources' code (file names + text without comments)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse_kernel(name: str):
    """(base name, integer/bool template arguments) from a demangled or an Itanium-mangled
    kernel name."""
    m = re.search(r"(k_[a-z0-9_]+)<([^>]*)>", name)
    if m:
        args = []
        for tok in m.group(2).split(","):
            tok = tok.strip()
            if re.fullmatch(r"-?\d+", tok):
                args.append(int(tok))
            elif tok in ("true", "false"):
                args.append(int(tok == "true"))
        return m.group(1), args
    m = re.search(r"\d+(k_[a-z0-9_]+)(I(.*?)E)?E?v", name)
    if m:
        base = m.group(1)
        args = [int(v) for v in re.findall(r"L[ib](-?\d+)E", m.group(3) or "")]
        return base, args
    m = re.search(r"(k_[a-z0-9_]+)", name)
    return (m.group(1) if m else name), []


def stage_of(name: str) -> str:
    base, args = parse_kernel(name)
    if base in ("k_router", "k_router_split", "k_router_epi", "k_router_tok"):
        return "route"
    if base in ("k_dispatch_count", "k_dispatch_scan", "k_dispatch_assign", "k_gather", "k_dispatch_small"):
        return "dispatch"
    if base == "k_route_dispatch_small":  # launched by moe_forward only (route epilogue + dispatch)
        return "forward"
    if base == "k_gemm_skinny_dual":  # dual-width skinny up-projection
        return "expert_up"
    if base in ("k_gemm_mixed", "k_gemm_mixed_reduce") and len(args) >= 2:  # <ACT, NB, ...>
        return "expert_up" if args[1] == 2 else "expert_down"
    if base in ("k_gemm_bf16", "k_gemm_tail_reduce", "k_gemm_streamk_reduce") and len(args) >= 3:
        return "expert_up" if args[2] == 2 else "expert_down"
    if base == "k_gemm_f32":
        return "expert_ffn"
    if base == "k_combine":
        return "combine"
    if base == "k_stats":
        return "stats"
    return "other"


def short_name(name: str) -> str:
    base, args = parse_kernel(name)
    return f"{base}<{', '.join(str(a) for a in args)}>" if args else base


def _one(pattern: str) -> str:
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise SystemExit(f"no file matches {pattern}")
    return files[0]


def kernel_stats(stats_csv: str):
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                         "total_us": float(r["TotalDurationNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3})
    return rows


def trace_last(trace_csv: str, last: int):
    """Per kernel name: average duration (us) of its last `last` dispatches, and its
    launch resources."""
    per = defaultdict(list)
    info = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
            info[r["Kernel_Name"]] = (r["Grid_Size_X"], r["Workgroup_Size_X"], r["VGPR_Count"], r["Accum_VGPR_Count"],
                                      r["LDS_Block_Size"], r["Scratch_Size"])
    out = {}
    for k, v in per.items():
        v.sort()
        tail = [d for _, d in v[-last:]]
        out[k] = (sum(tail) / len(tail), info[k])
    return out


def bench_stages(log: str):
    """The stage averages (ms) that bench.py measured with HIP events in the profiled run."""
    with open(log) as f:
        for line in reversed(f.read().splitlines()):
            if line.startswith("{") and '"stages_ms"' in line:
                return json.loads(line)["stages_ms"]
    return None


def cmd_stats(a):
    rows = kernel_stats(_one(os.path.join(a.dir, "**", "*kernel_stats.csv")) if os.path.isdir(a.dir) else a.dir)
    last = trace_last(_one(os.path.join(a.dir, "**", "*kernel_trace.csv")), a.last) if a.last else {}
    stage, stage_last = defaultdict(float), defaultdict(float)
    lines = [f"# Kernel durations: {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
             f"Kernel sources hash: `{source_hash()}`", "",
             f"`avg` is over every call (warm-up included); `timed avg` over the last {a.last} calls: for the "
             "stage kernels, the per-stage loop of bench.py whose HIP events give `bench events` below "
             "(kernels that only moe_forward launches: its timed loop)." if a.last else "", "",
             "| kernel | stage | calls | avg us | timed avg us | min us | max us | grid x wg | vgpr+agpr | lds B |",
             "|---|---|---:|---:|---:|---:|---:|---|---|---:|"]
    for r in sorted(rows, key=lambda r: STAGE_ORDER.index(stage_of(r["name"]))):
        st = stage_of(r["name"])
        tl, inf = last.get(r["name"], (float("nan"), ("", "", "", "", "", "")))
        lines.append(f"| `{short_name(r['name'])}` | {st} | {r['calls']} | {r['avg_us']:.2f} | {tl:.2f} | "
                     f"{r['min_us']:.2f} | {r['max_us']:.2f} | {inf[0]} x {inf[1]} | {inf[2]}+{inf[3]} | {inf[4]} |")
        # a kernel called fewer times than the timed loop (e.g. once while setting up) is
        # not one of the stage's timed kernels
        if st not in ("other", "forward", "stats") and (not a.last or r["calls"] >= a.last):
            stage[st] += r["avg_us"]
            stage_last[st] += tl
    bench = bench_stages(a.bench_log) if a.bench_log else None
    lines += ["", "Per-stage sums of the per-stage entry points' kernels (stage `forward`: kernels that only "
              "moe_forward launches, not summed; kernels called fewer times than the timed loop, e.g. once "
              "while setting up, not summed). `bench events` is what bench.py measured for the stage with "
              "HIP events on the launch stream in the same run.", "",
              "| stage | avg us | timed avg us | bench events us |", "|---|---:|---:|---:|"]
    for st in STAGE_ORDER:
        if st in stage:
            be = bench.get(st) * 1e3 if bench and st in bench else float("nan")
            lines.append(f"| {st} | {stage[st]:.2f} | {stage_last[st]:.2f} | {be:.2f} |")
    lines.append("")
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def counter_avgs(counter_csv: str, counter: str, with_counts: bool = False):
    """Average value of `counter` per dispatch, per kernel name (and the dispatch counts)."""
    tot, disp = defaultdict(float), defaultdict(set)
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            tot[r["Kernel_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    avg = {k: tot[k] / len(disp[k]) for k in tot}
    return (avg, {k: len(v) for k, v in disp.items()}) if with_counts else avg


def cmd_mfma(a):
    csv_path = _one(os.path.join(a.dir, "**", "*counter_collection.csv"))
    util = counter_avgs(csv_path, "MfmaUtil")
    flops = counter_avgs(csv_path, "MfmaFlopsBF16")
    useful = dict(kv.split("=") for kv in a.useful) if a.useful else {}
    lines = [f"# Matrix-core counters: {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
             f"Kernel sources hash: `{source_hash()}`", "",
             "Averages per dispatch over every call of the run. `MfmaUtil` = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(GRBM_GUI_ACTIVE x SIMDs) x 100; `bf16 flops` = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (all MFMAs "
             "issued, padding rows of partial tiles included); `useful` = the stage's algorithmic flops.", "",
             "| kernel | stage | MfmaUtil % | bf16 flops / dispatch | useful flops | executed / useful |",
             "|---|---|---:|---:|---:|---:|"]
    for k in sorted(util, key=lambda k: STAGE_ORDER.index(stage_of(k))):
        if flops.get(k, 0.0) <= 0.0:
            continue
        st = stage_of(k)
        u = float(useful[st]) if st in useful else float("nan")
        lines.append(f"| `{short_name(k)}` | {st} | {util[k]:.1f} | {flops[k]:.4g} | {u:.4g} | {flops[k] / u:.3f} |")
    lines.append("")
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def all_counter_avgs(counter_csv: str):
    """{kernel name: {counter: average value per dispatch}} over every counter of a run."""
    tot, disp = defaultdict(lambda: defaultdict(float)), defaultdict(lambda: defaultdict(set))
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            tot[r["Kernel_Name"]][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]][r["Counter_Name"]].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k][c]) for c, v in cs.items()} for k, cs in tot.items()}


# Ratios reported by `counters` when their operands were collected (each from one run).
DERIVED = [
    ("L2 hit %", "TCC_HIT_sum", "TCC_MISS_sum", lambda h, m: 100.0 * h / (h + m)),
    ("memory-side read latency (L2 cycles)", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", lambda l, n: l / n),
    ("TA busy / GUI active (summed over TA instances)", "TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE", lambda a, b: a / b),
    ("TA address stalled by L1 / TA busy %", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TA_TA_BUSY_sum",
     lambda a, b: 100.0 * a / b),
    ("LDS data FIFO full / SQ busy %", "SQ_LDS_DATA_FIFO_FULL", "SQ_BUSY_CYCLES", lambda a, b: 100.0 * a / b),
    ("LDS command FIFO full / SQ busy %", "SQ_LDS_CMD_FIFO_FULL", "SQ_BUSY_CYCLES", lambda a, b: 100.0 * a / b),
    ("LDS bank conflict / LDS active %", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", lambda a, b: 100.0 * a / b),
]


def cmd_counters(a):
    """Counter averages per dispatch of the stage kernels from one or more --pmc runs (one
    directory per run), with the ratios of DERIVED whose operands come from one run."""
    runs = [all_counter_avgs(_one(os.path.join(d, "**", "*counter_collection.csv"))) for d in a.dirs]
    kernels = sorted({k for r in runs for k in r if stage_of(k) in a.stages},
                     key=lambda k: (STAGE_ORDER.index(stage_of(k)), k))
    lines = [f"# Counters: {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
             f"Kernel sources hash: `{source_hash()}`", "",
             "Averages per dispatch over every call of each kernel in the run (one `--pmc` run per "
             "directory, counters from different runs are never combined in a ratio).", ""]
    for i, r in enumerate(runs):
        names = sorted({c for k in kernels if k in r for c in r[k]})
        if not names:
            continue
        lines += [f"Run {i + 1}: `{a.dirs[i]}`", "", "| kernel | stage | " + " | ".join(names) + " |",
                  "|---|---|" + "---:|" * len(names)]
        for k in kernels:
            if k not in r:
                continue
            lines.append(f"| `{short_name(k)}` | {stage_of(k)} | " +
                         " | ".join(f"{r[k].get(c, float('nan')):.6g}" for c in names) + " |")
        lines.append("")
        rows = []
        for title, x, y, f in DERIVED:
            if f is None:
                continue
            for k in kernels:
                if k in r and x in r[k] and y in r[k] and r[k][y] > 0:
                    rows.append(f"| `{short_name(k)}` | {title} | {f(r[k][x], r[k][y]):.4g} |")
        if rows:
            lines += ["| kernel | derived | value |", "|---|---|---:|"] + rows + [""]
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as fo:
            fo.write(text)
    print(text)


def cmd_traffic(a):
    fetch, nf = counter_avgs(_one(os.path.join(a.fetch, "**", "*counter_collection.csv")), "FETCH_SIZE", True)
    write = counter_avgs(_one(os.path.join(a.write, "**", "*counter_collection.csv")), "WRITE_SIZE")
    # a kernel dispatched far fewer times than the rest of its stage (e.g. once while the
    # bench sets up) is not one of the stage's kernels per launch
    most = defaultdict(int)
    for k, n in nf.items():
        most[stage_of(k)] = max(most[stage_of(k)], n)
    cf = counter_avgs(_one(os.path.join(a.copy_fetch, "**", "*counter_collection.csv")), "FETCH_SIZE")
    cw = counter_avgs(_one(os.path.join(a.copy_write, "**", "*counter_collection.csv")), "WRITE_SIZE")
    # the copy run launches one kernel kind: the largest per-dispatch figure is the copy
    copy_bytes = a.copy_mib * 2 ** 20
    f_fetch = copy_bytes / (max(cf.values()) * 1024.0)
    f_write = copy_bytes / (max(cw.values()) * 1024.0)
    stages = defaultdict(lambda: {"fetch_kib": 0.0, "write_kib": 0.0, "kernels": []})
    for k in sorted(set(fetch) | set(write)):
        st = stage_of(k)
        if st == "other" or 2 * nf.get(k, 0) < most[st]:
            continue
        stages[st]["fetch_kib"] += fetch.get(k, 0.0)
        stages[st]["write_kib"] += write.get(k, 0.0)
        stages[st]["kernels"].append(short_name(k))
    out = {"workload": a.workload, "source_hash": source_hash(), "copy_mib": a.copy_mib,
           "copy_kind": a.copy_kind, "scale_fetch": f_fetch, "scale_write": f_write,
           "what": "bytes through the L2's memory-side interface per launch (L2 misses and write-backs, served "
                   "by the Infinity Cache or HBM): FETCH_SIZE and WRITE_SIZE scaled by the calibration copy",
           "command": a.cmd, "stages": {}}
    for st, v in stages.items():
        mem = v["fetch_kib"] * 1024.0 * f_fetch + v["write_kib"] * 1024.0 * f_write
        out["stages"][st] = {"kernels": v["kernels"], "fetch_kib_per_launch": v["fetch_kib"],
                             "write_kib_per_launch": v["write_kib"], "memory_bytes_per_launch": mem}
    text = json.dumps(out, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def main():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = p.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir", help="rocprofv3 output directory (or the kernel_stats.csv itself)")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True, help="the command that produced the profile")
    s.add_argument("--last", type=int, default=0, help="also average the last N calls of each kernel")
    s.add_argument("--bench-log", help="log of the profiled bench.py run (its JSON line)")
    s.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+", help="rocprofv3 --pmc output directories, one per run")
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--stages", nargs="+", default=["expert_up", "expert_down"])
    c.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--copy-kind", default="lds", help="the calibration copy's read path (bench.py --copy-kind)")
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("dir", help="rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 output directory")
    m.add_argument("--title", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--useful", nargs="*", help="stage=flops pairs (useful flops per launch)")
    m.add_argument("--out")
    a = p.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma, "counters": cmd_counters}[a.cmd_name](a)


if __name__ == "__main__":
    main()
