"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

Usage:
  python parameter_efficient_fine_nf4_amd/profile_summary.py stats \\
      --dir D --name N --main-dispatches K [--skip S] --cmd "..." --out profiles/X.md
  python parameter_efficient_fine_nf4_amd/profile_summary.py traffic \\
      --fetch-dir D1 --write-dir D2 --name N --workload W --cmd-fetch "..." \\
      --cmd-write "..." --out profiles/Y.md --json profiles/hbm_traffic.json

stats    per-kernel launch counts and durations from a --kernel-trace --stats
         run: the profiler's own table, plus the mean over dispatches
         [skip, skip + K) of each library kernel in launch order (the timed
         pass of a run that executes its main workload first).
traffic  per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of every kernel from two
         --pmc runs, each scaled by the factor that maps the same counter of
         the reference streaming kernel (torch.neg over 256 MiB: 256 MiB read
         and 256 MiB written per launch) onto its known traffic.  The JSON
         record of each library kernel carries the hash of its source file so
         that a changed kernel does not inherit old counters.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20

# library kernel symbol -> (short name, source file)
KERNELS = {
    "k_fwd8": ("fwd_rich", "gemm_fwd.hip"),
    "k_fwd_rich": ("fwd_rich", "gemm_fwd.hip"),
    "k_fwd_decode_finish": ("fwd_decode_finish", "gemm_fwd.hip"),
    "k_fwd_decode": ("fwd_decode", "gemm_fwd.hip"),
    "k_fwd_dec": ("fwd_decode", "gemm_fwd.hip"),
    "k_dx8": ("dx", "gemm_dx.hip"),
    "k_dx": ("dx", "gemm_dx.hip"),
    "k_lora_proj_finish": ("lora_proj_finish", "lora.hip"),
    "k_proj": ("lora_proj", "lora.hip"),
    "k_proj2": ("lora_proj", "lora.hip"),
    "k_tokred": ("token_reduce", "lora.hip"),
    "k_prep": ("prep_adapters", "lora.hip"),
    "k_drop_input": ("drop_input", "lora.hip"),
    "k_adam": ("adam", "optim.hip"),
    "k_sum_splits": ("sum_splits", "gemm_fwd.hip"),
    "k_merge": ("merge", "merge.hip"),
    "k_quant_blocks": ("quant_blocks", "quant.hip"),
    "k_group_sums": ("quant_group_sums", "quant.hip"),
    "k_mean": ("quant_mean", "quant.hip"),
    "k_dq": ("quant_dq", "quant.hip"),
}


def short_name(kernel_name: str) -> str:
    base = kernel_name.split("(")[0]
    base = base.replace("void ", "").strip()
    sym = base.split("::")[-1].split("<")[0]
    if sym in KERNELS:
        return KERNELS[sym][0]
    if "neg" in kernel_name and "elementwise" in kernel_name.lower():
        return "reference_stream_neg"
    return base[:60]


def src_sha(short: str) -> str | None:
    for sym, (name, f) in KERNELS.items():
        if name == short:
            with open(os.path.join(PKG, "csrc", f), "rb") as fh:
                return hashlib.sha256(fh.read()).hexdigest()[:16]
    return None


def find(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def cmd_stats(a) -> None:
    stats = list(csv.DictReader(open(find(a.dir, f"{a.name}_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(find(a.dir, f"{a.name}_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    for r in trace:
        per[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "Command (from the repository root):", "",
             "```", a.cmd, "```", "",
             "## Profiler summary (all dispatches of the run)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    lo, hi = a.skip, a.skip + a.main_dispatches
    lines += ["", f"## Main workload: dispatches {lo}..{hi - 1} of each library kernel "
                  f"(in launch order; the timed pass of the run)", "",
              "| kernel | dispatches | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for n in sorted(per, key=lambda n: -sum(per[n])):
        if not any(n == v[0] for v in KERNELS.values()):
            continue
        v = per[n][lo:hi] or per[n]
        lines.append(f"| {n} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(d: str, name: str, counter: str) -> dict:
    rows = list(csv.DictReader(open(find(d, f"{name}_counter_collection.csv"))))
    per = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def cmd_traffic(a) -> None:
    fetch = counters(a.fetch_dir, a.name, "FETCH_SIZE")
    write = counters(a.write_dir, a.name, "WRITE_SIZE")
    ref = "reference_stream_neg"
    if ref not in fetch or ref not in write:
        raise SystemExit("the reference streaming kernel is missing from the counter runs")
    f_fetch = COPY_BYTES / (fetch[ref] * 1024.0)
    f_write = COPY_BYTES / (write[ref] * 1024.0)
    lines = [f"# HBM traffic per dispatch: {a.workload}", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc), each run on its own:", "",
             "```", a.cmd_fetch, a.cmd_write, "```", "",
             f"Scale factors from the reference streaming kernel (256 MiB read + 256 MiB written): "
             f"FETCH {fetch[ref]:.0f} KiB -> x{f_fetch:.4f}, WRITE {write[ref]:.0f} KiB -> x{f_write:.4f}.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes / dispatch | MB |",
             "|---|---:|---:|---:|---:|"]
    db = {}
    if os.path.exists(a.json):
        db = json.load(open(a.json))
    for n in sorted(fetch, key=lambda n: -fetch[n]):
        if n not in write:
            continue
        b = fetch[n] * 1024.0 * f_fetch + write[n] * 1024.0 * f_write
        lines.append(f"| {n} | {fetch[n]:.0f} | {write[n]:.0f} | {b:.0f} | {b / 1e6:.2f} |")
        sha = src_sha(n)
        if sha is not None:
            db[f"{n}@{a.workload}"] = {"bytes_per_launch": round(b), "fetch_kib": round(fetch[n], 1),
                                       "write_kib": round(write[n], 1), "fetch_factor": round(f_fetch, 5),
                                       "write_factor": round(f_write, 5), "src_sha": sha}
    open(a.out, "w").write("\n".join(lines) + "\n")
    with open(a.json, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print("\n".join(lines))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--name", required=True)
    s.add_argument("--main-dispatches", type=int, required=True)
    s.add_argument("--skip", type=int, default=0)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-dir", required=True)
    t.add_argument("--write-dir", required=True)
    t.add_argument("--name", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--json", required=True)
    a = ap.parse_args()
    cmd_stats(a) if a.action == "stats" else cmd_traffic(a)


if __name__ == "__main__":
    main()
