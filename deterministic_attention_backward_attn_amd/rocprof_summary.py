"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m deterministic_attention_backward_attn_amd.rocprof_summary stats \\
      --csv <dir>/<prefix>_kernel_stats.csv --cmd "<command>" --out profiles/<name>.md \\
      [--trace <dir>/<prefix>_kernel_trace.csv --blocks atomic,naive,descending,shift \\
       --block-size W+K]

  python -m deterministic_attention_backward_attn_amd.rocprof_summary traffic \\
      --fetch-csv <dir>/<prefix>_counter_collection.csv \\
      --write-csv <dir>/<prefix>_counter_collection.csv \\
      --copy-bytes N [--kernel NAME|NAME] --flops F [--dispatches A:B] \\
      --cmd-fetch "<command>" --cmd-write "<command>" --out profiles/<name>.md

With --trace, the backward kernel's dispatches (in dispatch order) are cut
into consecutive blocks of --block-size, one per name in --blocks (bench.py
times its schedules one after another, W warm-up plus K timed launches
each), and per-schedule durations are listed: the ordered schedules share
one kernel instantiation, so the statistics table alone mixes them.

  python -m deterministic_attention_backward_attn_amd.rocprof_summary counters \\
      --csv <dir>/<prefix>_counter_collection.csv --cmd "<command>" \\
      --blocks atomic,descending --block-size K --out profiles/<name>.md

The counters summary lists the SQ counters of one rocprofv3 --pmc pass per
schedule (backward dispatches cut into blocks as above) with derived
figures: MFMA busy share (MFMA-busy cycles over 1024 SIMDs / busy cycles
over 32 shader engines), LDS bank-conflict share of LDS-active cycles, and
the share of wave cycles spent in s_waitcnt.

  python -m deterministic_attention_backward_attn_amd.rocprof_summary phases \\
      --log <bench output with --phases> --cmd "<command>" --out profiles/<name>.md

The phases summary tabulates the per-phase shares of wave cycles that
bench.py --phases reads from the backward's phase timer (a test hook; its
clock reads slow the launch, so shares, not times, are the result), one
column per schedule, with the kernel times of the same run.

The traffic summary scales each kernel's FETCH_SIZE / WRITE_SIZE (KiB per
dispatch) by the factor that makes the same counter read the known size of a
plain device copy run in the same process, and records the hash of the
backward kernel's sources so that a reader can tell whether the figure still
describes the current kernel.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# every source of the backward kernels' translation units (the one-stage
# kernel and the two-stage pipeline that bf16 with d = 128 runs) and what
# they include
KERNEL_SOURCES = ["deterministic_attention_backward_attn_amd/csrc/kernels/attn_bwd.hip",
                  "deterministic_attention_backward_attn_amd/csrc/kernels/attn_bwd_pipe.hip",
                  "deterministic_attention_backward_attn_amd/csrc/kernels/common.hpp",
                  "deterministic_attention_backward_attn_amd/csrc/kernels/launch.hpp",
                  "deterministic_attention_backward_attn_amd/csrc/kernels/placement.hpp"]
# names of the backward kernels' dispatches
BWD_KERNELS = ("bwd_kernel", "bwd_pipe_kernel", "bwd_pair_kernel")


def is_bwd(name: str) -> bool:
    return any(k in name for k in BWD_KERNELS)


def kernel_source_hash() -> str:
    """Hash of the backward kernel's sources and its device compile flags."""
    from deterministic_attention_backward_attn_amd import build as B
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(B.DEVICE + B.PER_FILE.get("kernels/attn_bwd.hip", [])
                      + B.PER_FILE.get("kernels/attn_bwd_pipe.hip", [])).encode())
    return h.hexdigest()[:16]


def _short(name: str, n: int = 110) -> str:
    name = name.replace("dash::", "")
    return name if len(name) <= n else name[: n - 3] + "..."


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{args.cmd}`", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |",
             "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    if args.trace:
        rows = sorted(csv.DictReader(open(args.trace)), key=lambda r: int(r["Dispatch_Id"]))
        bwd = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
               for r in rows if is_bwd(r["Kernel_Name"])]
        names = [b for b in args.blocks.split(",") if b]
        if len(bwd) != len(names) * args.block_size:
            raise SystemExit(f"{len(bwd)} backward dispatches, expected "
                             f"{len(names)} x {args.block_size}")
        lines += ["", "Backward kernel per schedule (dispatches in order, "
                  f"{args.block_size} per schedule; 'timed avg' leaves out the first "
                  f"{args.warmup}, the warm-up launches):", "",
                  "| schedule | dispatches | avg us | timed avg us | min us | max us |",
                  "|---|---|---|---|---|---|"]
        for i, name in enumerate(names):
            d = bwd[i * args.block_size:(i + 1) * args.block_size]
            timed = d[args.warmup:] or d
            lines.append(f"| {name} | {len(d)} | {statistics.mean(d):.1f} | "
                         f"{statistics.mean(timed):.1f} | {min(d):.1f} | {max(d):.1f} |")
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
    _write(args.out, lines)


def _per_dispatch(path, counter):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        out.setdefault(key, [r["Kernel_Name"], 0.0, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        out[key][1] += float(r["Counter_Value"])
    return out


def traffic(args):
    fetch = _per_dispatch(args.fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(args.write_csv, "WRITE_SIZE")

    def copy_kib(d):
        # the largest elementwise copy dispatch is the calibration copy
        cands = [v for v in d.values() if "copy" in v[0].lower() or "elementwise" in v[0].lower()]
        if not cands:
            raise SystemExit("no copy dispatch found for calibration")
        return max(cands, key=lambda v: v[1])[1]

    known_kib = args.copy_bytes / 1024.0
    f_fac = known_kib / copy_kib(fetch)
    w_fac = known_kib / copy_kib(write)
    def pick(d, i):
        vals = [d[k][i] for k in sorted(d) if any(n in d[k][0] for n in args.kernel.split("|"))]
        if args.dispatches:
            a, b = (int(x) for x in args.dispatches.split(":"))
            vals = vals[a:b]
        return vals

    fk, wk, dur = pick(fetch, 1), pick(write, 1), pick(fetch, 2)
    if not fk or not wk:
        raise SystemExit(f"no dispatch of {args.kernel}")
    fetch_b = statistics.mean(fk) * f_fac * 1024
    write_b = statistics.mean(wk) * w_fac * 1024
    lines = ["# HBM traffic of the backward kernel (rocprofv3 counters)", "",
             f"FETCH_SIZE pass: `{args.cmd_fetch}`", "",
             f"WRITE_SIZE pass: `{args.cmd_write}`", "",
             f"Calibration: a plain device copy of {args.copy_bytes} bytes in the same process; "
             f"FETCH_SIZE factor {f_fac:.4f}, WRITE_SIZE factor {w_fac:.4f} "
             f"(known bytes / counter reading).", "",
             f"Dispatches of `{args.kernel}`: {len(fk)}"
             + (f" (numbers {args.dispatches} of the run, in dispatch order)" if args.dispatches else "")
             + f"; raw FETCH_SIZE {statistics.mean(fk):.0f} KiB, "
             f"raw WRITE_SIZE {statistics.mean(wk):.0f} KiB per dispatch.", "",
             f"fetch_bytes_per_launch: {fetch_b:.6g}",
             f"write_bytes_per_launch: {write_b:.6g}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.6g}"]
    if args.flops:
        lines.append(f"arithmetic_intensity_flop_per_byte: {args.flops / (fetch_b + write_b):.1f}")
    if dur:
        lines.append(f"counter_pass_avg_duration_us: {statistics.mean(dur) / 1e3:.1f} "
                     "(counter passes serialise dispatches; not a timing figure)")
    lines += [f"kernel_source_sha256: {kernel_source_hash()}", ""]
    _write(args.out, lines)


def counters(args):
    per = {}
    for r in csv.DictReader(open(args.csv)):
        if not any(k in r["Kernel_Name"] for k in args.kernel.split("|")):
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)
    names = [b for b in args.blocks.split(",") if b]
    if len(ids) != len(names) * args.block_size:
        raise SystemExit(f"{len(ids)} dispatches, expected {len(names)} x {args.block_size}")
    ctrs = sorted({c for d in per.values() for c in d})
    lines = [f"# rocprofv3 SQ counters of `{args.kernel}`", "",
             f"Command: `{args.cmd}`", "",
             f"Per schedule: mean over its {args.block_size} dispatches (dispatch order).", "",
             "| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    means = []
    for i, _ in enumerate(names):
        blk = ids[i * args.block_size:(i + 1) * args.block_size]
        means.append({c: statistics.mean(per[d].get(c, 0.0) for d in blk) for c in ctrs})
    for c in ctrs:
        lines.append(f"| {c} | " + " | ".join(f"{m[c]:.4g}" for m in means) + " |")

    def ratio(m, a, b, k=1.0):
        return f"{m[a] / (k * m[b]):.3f}" if a in m and b in m and m[b] else "n/a"
    lines += ["", "| derived | " + " | ".join(names) + " |", "|---|" + "---|" * len(names),
              "| MFMA busy share | " + " | ".join(
                  ratio(m, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", 32.0) for m in means) + " |",
              "| LDS bank-conflict share of LDS-active cycles | " + " | ".join(
                  ratio(m, "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE") for m in means) + " |",
              "| wave cycles in s_waitcnt | " + " | ".join(
                  ratio(m, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES") for m in means) + " |",
              ""]
    if "bwd" in args.kernel:
        lines += [f"kernel_source_sha256: {kernel_source_hash()}", ""]
    _write(args.out, lines)


def _write(path, lines):
    text = "\n".join(lines)
    if path:
        with open(path, "w") as f:
            f.write(text)
    print(text)


def phases(args):
    import json
    line = [ln for ln in open(args.log) if ln.startswith('{"metric"')][-1]
    run = json.loads(line)
    scheds = [s for s, r in run["schedules"].items() if "phases" in r]
    names = list(run["schedules"][scheds[0]]["phases"])
    lines = ["# Phase shares of the backward kernel's wave cycles", "",
             f"Command: `{args.cmd}`", "",
             f"Workload: {run['config']['workload']}"
             + (f", backward layout: {run['config']['layout']}" if "layout" in run["config"] else "")
             + ".  Shares of each wave's cycles per phase "
             "of its Q sub-tiles, from one extra launch per schedule with the phase timer "
             "(its clock reads slow that launch; shares, not times).", "",
             "| phase | " + " | ".join(scheds) + " |",
             "|---|" + "---|" * len(scheds)]
    for n in names:
        lines.append(f"| {n} | " + " | ".join(f"{run['schedules'][s]['phases'][n]:.3f}"
                                              for s in scheds) + " |")
    # the 8-wave layouts time each role's waves separately ("A: ...", "B: ...")
    groups = sorted({n.split(": ")[0] for n in names if ": " in n}) or [None]
    for g in groups:
        keys = [n for n in names if g is None or n.startswith(g + ": ")]
        lines.append(f"| sum{'' if g is None else ' ' + g} | " + " | ".join(
            f"{sum(run['schedules'][s]['phases'][k] for k in keys):.3f}" for s in scheds) + " |")
    lines.append("| kernel ms (timed launches, no timer) | " + " | ".join(
        f"{run['schedules'][s]['kernel_ms']:.3f}" for s in scheds) + " |")
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
    text = "\n".join(lines)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out")
    s.add_argument("--trace")
    s.add_argument("--blocks", default="atomic,naive,descending,shift")
    s.add_argument("--block-size", type=int, default=0)
    s.add_argument("--warmup", type=int, default=0,
                   help="leading dispatches of each block that were warm-up launches")
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out")
    c.add_argument("--kernel", default="|".join(BWD_KERNELS))
    c.add_argument("--blocks", default="atomic,descending")
    c.add_argument("--block-size", type=int, default=3)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-csv", required=True)
    t.add_argument("--write-csv", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", default="|".join(BWD_KERNELS))
    t.add_argument("--flops", type=float, default=0.0)
    t.add_argument("--dispatches", default="",
                   help="a:b = only the backward dispatches a..b-1 (dispatch order), e.g. one "
                        "schedule's block when the run timed several")
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out")
    ph = sub.add_parser("phases")
    ph.add_argument("--log", required=True)
    ph.add_argument("--cmd", required=True)
    ph.add_argument("--out")
    args = ap.parse_args(argv)
    {"stats": stats, "traffic": traffic, "counters": counters, "phases": phases}[args.mode](args)


if __name__ == "__main__":
    main(sys.argv[1:])
