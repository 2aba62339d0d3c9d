"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

Usage (from the repository root; D is the directory rocprofv3 wrote to):
  python parameter_efficient_fine_nf4_amd/profile_summary.py trace --dir D [--bench-log LOG]
  python parameter_efficient_fine_nf4_amd/profile_summary.py traffic --fetch-dir D1 --write-dir D2
  python parameter_efficient_fine_nf4_amd/profile_summary.py counters --dirs DA DB DC
  python parameter_efficient_fine_nf4_amd/profile_summary.py decode-counters --dir D
  python parameter_efficient_fine_nf4_amd/profile_summary.py fetch --dir D

trace     a --kernel-trace --stats run of bench.py: per-kernel durations of
          the headline leg's 20 timed steps and of its 20-step kernel-timing
          pass (after 5 warm-up steps; five dispatches per step), with
          --bench-log the bench line of that run set against them, and the
          profiler's own table over the whole run
          -> profiles/kernel_trace_bench_d4096_k4096_M4096_r16.md
traffic   FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two --pmc runs of
          profile_run.py --what train,decode,decode_rot,copy, each scaled by
          the factor that maps the same counter of the reference streaming
          kernel (torch.neg over 256 MiB: 256 MiB read and 256 MiB written
          per launch) onto its known traffic; the training step's kernels,
          the first three decode calls and the 192 rotated ones are kept
          apart.  The JSON record of each library kernel carries the hash of
          its source file, so a changed kernel does not inherit old counters.
          -> profiles/hbm_traffic.json, profiles/hbm_traffic_<workload>.md
counters  three --pmc runs of profile_run.py --what train (the counter sets
          in COUNTER_PASSES): MFMA busy cycles, instruction mix, VALU/MFMA
          co-issue and LDS stalls per kernel, with the derived shader clock
          and MFMA utilisation
          -> profiles/mfma_counters_d4096_k4096_M4096_r16.md
decode-counters
          one --pmc run of profile_run.py --what decode_rot (DECODE_COUNTERS):
          per-wave instruction counts and wait shares of the decode kernels
          -> profiles/decode_counters_d4096_k4096_M16_r16_rot64.md
fetch     one --pmc run of profile_run.py --what train,decode_rot
          (FETCH_COUNTERS): read requests from each CU's vector L1 to L2,
          their mean latency and L2 hit rate, and from those (Little's law)
          the requests each CU keeps in flight, next to the bytes each CU
          must read (set out per kernel in CU_READ_BYTES)
          -> profiles/l1_fetch_counters.md
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
TRAIN = "d4096_k4096_M4096_r16"
DECODE = "d4096_k4096_M16_r16"
DECODE_ROT = "d4096_k4096_M16_r16_rot64"
MERGE = "d8192_k8192_r64_merge"

PROFILE_CMD = ("cd /tmp && TMPDIR=/tmp timeout -s KILL {t} rocprofv3 --pmc {c} -d <repo>/gpurun_out/{d} -o run "
               "--output-format csv -- python3 <repo>/parameter_efficient_fine_nf4_amd/profile_run.py {args}")
TRAFFIC_ARGS = "--what train,decode,decode_rot,copy,merge --steps 3"
COUNTER_ARGS = "--what train --steps 3"
COUNTER_PASSES = {
    "pmcA": "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_LDS "
            "SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE",
    "pmcB": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_ANY "
            "SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT",
    "pmcC": "SQ_ACTIVE_INST_LDS SQ_INST_CYCLES_VMEM_RD SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_CYCLES "
            "SQ_BUSY_CU_CYCLES SQ_WAVES SQ_INSTS_VMEM_RD",
}

# library kernel symbol (as it appears before "(") -> (short name, source file)
KERNELS = [
    ("k_fwd8", "fwd_rich", "gemm_fwd.hip"),
    ("k_fwd_rich", "fwd_rich", "gemm_fwd.hip"),
    ("k_fwd_decode_finish", "fwd_decode_finish", "gemm_fwd.hip"),
    ("k_fwd_decode", "fwd_decode", "gemm_fwd.hip"),
    ("k_fwd_dec1s", "fwd_decode", "gemm_fwd.hip"),
    ("k_fwd_dec1", "fwd_decode", "gemm_fwd.hip"),
    ("k_fwd_dec", "fwd_decode", "gemm_fwd.hip"),
    ("k_dx8", "dx", "gemm_dx.hip"),
    ("k_dx", "dx", "gemm_dx.hip"),
    ("k_lora_proj_finish", "lora_proj_finish", "lora.hip"),
    ("k_proj<1, false>", "lora_proj_T", "lora.hip"),
    ("k_proj<1, true>", "lora_proj_U", "lora.hip"),
    ("k_proj2", "lora_proj", "lora.hip"),
    ("k_proj", "lora_proj", "lora.hip"),
    ("k_tokred", "token_reduce", "lora.hip"),
    ("k_prep", "prep_adapters", "lora.hip"),
    ("k_drop_input", "drop_input", "lora.hip"),
    ("k_adam", "adam", "optim.hip"),
    ("k_sum_splits", "sum_splits", "gemm_fwd.hip"),
    ("k_merge_runs", "merge", "merge.hip"),
    ("k_merge", "merge", "merge.hip"),
    ("k_quant_blocks", "quant_blocks", "quant.hip"),
    ("k_group_sums", "quant_group_sums", "quant.hip"),
    ("k_mean", "quant_mean", "quant.hip"),
    ("k_dq", "quant_dq", "quant.hip"),
]


def symbol(kernel_name: str) -> str:
    return kernel_name.split("(")[0].replace("void ", "").replace("qlora::", "").strip()


def short_name(kernel_name: str) -> str | None:
    sym = symbol(kernel_name)
    for key, name, _ in KERNELS:
        if sym == key or sym.startswith(key + "<") or (key.endswith(">") and sym == key):
            return name
    if "neg_kernel" in kernel_name:
        return "reference_stream_neg"
    return None


def src_sha(short: str) -> str | None:
    for _, name, f in KERNELS:
        if name == short:
            with open(os.path.join(PKG, "csrc", f), "rb") as fh:
                return hashlib.sha256(fh.read()).hexdigest()[:16]
    return None


def find(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def write(path: str, lines: list[str]) -> None:
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", path)


# ------------------------------------------------------------------ trace --

def cmd_trace(a) -> None:
    rows = list(csv.DictReader(open(find(a.dir, "*kernel_trace.csv"))))
    stats = list(csv.DictReader(open(find(a.dir, "*kernel_stats.csv"))))
    first = next(i for i, r in enumerate(rows) if symbol(r["Kernel_Name"]).startswith("k_fwd8"))

    def section(lo: int, hi: int, title: str) -> list[str]:
        part = rows[first + lo:first + hi]
        per = collections.OrderedDict()
        for r in part:
            per.setdefault((symbol(r["Kernel_Name"]), r["Grid_Size_X"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        n = (hi - lo) // 5
        span = (int(part[-1]["End_Timestamp"]) - int(part[0]["Start_Timestamp"])) / 1e3 / n
        busy = sum(sum(v) for v in per.values()) / n
        out = [f"## {title}", "", "| kernel | grid threads | dispatches | avg us | min us | max us |",
               "|---|---:|---:|---:|---:|---:|"]
        for (nm, g), v in per.items():
            out.append(f"| {nm} | {g} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        out += ["", f"Per step: {busy:.1f} us of kernel time, {span:.1f} us from the first kernel's start to the "
                f"last one's end.", ""]
        return out

    L = [f"# rocprofv3 kernel trace: bench.py, QLoRA linear d = k = 4096, M = 4096, r = 16 fwd+bwd", "",
         "Command (from the repository root), then "
         "`profile_summary.py trace --dir gpurun_out/prof_bench --bench-log gpurun_out/trace_bench.log`:", "",
         "```",
         "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <repo>/gpurun_out/prof_bench -o bench "
         "--output-format csv -- python3 <repo>/bench.py --steps 20 --warmup 5 --no-cpu-baseline --decode-reps 2 "
         "> <repo>/gpurun_out/trace_bench.log",
         "```", "",
         "The headline leg runs 5 warm-up steps, the 20 timed steps, then 20 more steps with the library's per-kernel "
         "HIP-event timing on (the kernel-timing pass: the source of the bench line's per-kernel times and "
         "roofline).", ""]
    L += section(25, 125, "Headline workload: the 20 timed steps")
    L += section(125, 225, "Headline workload: the 20 steps of the kernel-timing pass")
    if a.bench_log:
        L += bench_vs_trace(a.bench_log, rows[first + 125:first + 225])
    L += ["## Profiler summary (all dispatches of the run: every leg and shape)", "",
          "| kernel | calls | avg us | min us | max us | % time |", "|---|---:|---:|---:|---:|---:|"]
    for s in stats[:30]:
        L.append(f"| {symbol(s['Name'])[:60]} | {s['Calls']} | {float(s['AverageNs']) / 1e3:.2f} | "
                 f"{int(s['MinNs']) / 1e3:.2f} | {int(s['MaxNs']) / 1e3:.2f} | {float(s['Percentage']):.2f} |")
    write(os.path.join(PROFILES, f"kernel_trace_bench_{TRAIN}.md"), L)


def bench_vs_trace(log: str, part: list) -> list[str]:
    """The bench line's per-kernel times (HIP events around each launch) next
    to the profiler's durations of the same launches."""
    line = next(ln for ln in open(log) if ln.startswith("{") and '"metric"' in ln)
    rec = json.loads(line)
    ev = rec["kernels_us_per_launch"]
    per = collections.defaultdict(list)
    for r in part:
        nm = short_name(r["Kernel_Name"])
        if nm in ("lora_proj_T", "lora_proj_U"):
            nm = "lora_proj"
        per[nm].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["## The bench line of this run against the trace", "",
           "Per-kernel times of the bench line printed by this same run (the HIP event pair each launch of the "
           "kernel-timing pass carries, stamped by hipExtLaunchKernel on the launch stream) next to the "
           "profiler's kernel durations of those launches.", "",
           "| kernel | bench line us | trace us | bench - trace us | bench / trace |", "|---|---:|---:|---:|---:|"]
    gaps = []
    for nm, us in ev.items():
        if per.get(nm):
            t = statistics.mean(per[nm])
            gaps.append(us - t)
            out.append(f"| {nm} | {us:.2f} | {t:.2f} | {us - t:.2f} | {us / t:.3f} |")
    rf = rec["roofline"]
    out += ["", f"The event pair spans {min(gaps):.1f} to {max(gaps):.1f} us more than the profiler's kernel "
            "duration whatever the kernel's length: a fixed cost per launch, so the bench line's rates are the "
            "lower of the two.", "",
            f"Bench line roofline ({rf['kernel']}): {rf['achieved']:.1f} {rf['unit']} of {rf['peak']:.1f}, "
            f"frac {rf['frac']:.4f} over {rf['us_per_launch']:.2f} us per launch.", ""]
    return out


# ---------------------------------------------------------------- traffic --

def nf4_bytes(d: int, k: int) -> int:
    nb = d * k // 64
    return d * k // 2 + nb + 4 * ((nb + 255) // 256) + 4


def cmd_traffic(a) -> None:
    def load(d):
        out = collections.OrderedDict()
        for r in csv.DictReader(open(find(d, "*counter_collection.csv"))):
            out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
        return out

    F, W = load(a.fetch_dir), load(a.write_dir)
    if list(F) != list(W):
        raise SystemExit("the two passes saw different dispatches")
    neg = [(F[i][1], W[i][1]) for i in F if short_name(F[i][0]) == "reference_stream_neg"]
    copy_kib = 256 * 1024  # KiB read, and written, per launch of the reference kernel
    ff = copy_kib / statistics.mean(f for f, _ in neg)
    wf = copy_kib / statistics.mean(w for _, w in neg)
    groups = collections.defaultdict(list)
    ndec = nneg = 0
    for i, (n, fv) in F.items():
        s = short_name(n)
        if s is None:
            continue
        ndec += s == "fwd_decode"
        nneg += s == "reference_stream_neg"
        if s.startswith("fwd_decode"):
            wl = DECODE if ndec <= 3 else DECODE_ROT
        else:  # the merge workload runs after the reference kernel
            wl = MERGE if nneg == len(neg) and s != "reference_stream_neg" else TRAIN
        groups[(s, wl)].append((fv, W[i][1]))
    nf4 = nf4_bytes(4096, 4096)
    act = 4096 * 4096 * 2
    alg = {("fwd_rich", TRAIN): nf4 + 2 * act + 2 * 4096 * 16 * 2,
           ("dx", TRAIN): nf4 + 2 * act + 2 * 4096 * 16 * 2,
           ("lora_proj_T", TRAIN): act + 3 * 4096 * 16 * 2,
           ("lora_proj_U", TRAIN): act + 5 * 4096 * 16 * 2,
           ("token_reduce", TRAIN): 2 * act + 4 * 4096 * 16 * 2,
           ("merge", MERGE): nf4_bytes(8192, 8192) + 2 * 8192 * 8192 + 2 * 64 * (8192 + 8192)}
    pair = nf4 + 2 * 16 * 4096 * 2 + 2 * 4096 * 16 * 2  # decode call: NF4 + X + Y + A + B
    rec, tables = {}, collections.defaultdict(list)
    for (s, wl), v in sorted(groups.items()):
        fk, wk = statistics.mean(x for x, _ in v), statistics.mean(y for _, y in v)
        by = int(round(fk * 1024 * ff + wk * 1024 * wf))
        sha = src_sha(s)
        if sha is not None:
            rec[f"{s}@{wl}"] = {"bytes_per_launch": by, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                "fetch_factor": round(ff, 5), "write_factor": round(wf, 5), "src_sha": sha,
                                "dispatches": len(v)}
        tables[TRAIN if s == "reference_stream_neg" else wl].append((s, len(v), fk, wk, by, alg.get((s, wl))))
    with open(os.path.join(PROFILES, "hbm_traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print("wrote profiles/hbm_traffic.json")
    for wl, rows in tables.items():
        L = [f"# HBM traffic per dispatch: {wl}", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the dispatches), one rocprofv3 pass each, then "
             "`profile_summary.py traffic --fetch-dir gpurun_out/pmc_FETCH_SIZE --write-dir gpurun_out/pmc_WRITE_SIZE`:",
             "", "```", PROFILE_CMD.format(t=150, c="FETCH_SIZE", d="pmc_FETCH_SIZE", args=TRAFFIC_ARGS),
             PROFILE_CMD.format(t=150, c="WRITE_SIZE", d="pmc_WRITE_SIZE", args=TRAFFIC_ARGS), "```", "",
             f"Scale factors from the reference streaming kernel (torch.neg over 256 MiB bf16: 256 MiB read + "
             f"256 MiB written per launch): FETCH x{ff:.4f}, WRITE x{wf:.4f}.  FETCH_SIZE counts L2 misses, which the "
             f"256 MB last-level cache may still serve.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB / dispatch | algorithmic MB | ratio |",
             "|---|---:|---:|---:|---:|---:|---:|"]
        for s, n, fk, wk, by, al in sorted(rows, key=lambda t: -t[4]):
            L.append(f"| {s} | {n} | {fk:.0f} | {wk:.0f} | {by / 1e6:.2f} | "
                     f"{'' if al is None else f'{al / 1e6:.2f}'} | {'' if al is None else f'{by / al:.2f}'} |")
        if wl in (DECODE, DECODE_ROT):
            names = [t[0] for t in rows if t[0] in ("fwd_decode", "fwd_decode_finish")]
            call = sum(t[4] for t in rows if t[0] in names)
            L += ["", f"One forward call ({' + '.join(names)}): {call / 1e6:.2f} MB moved against "
                  f"{pair / 1e6:.2f} MB algorithmic (NF4 weight + X + Y + A + B): x{call / pair:.2f}."]
        if wl == MERGE:
            L += ["", "Algorithmic: the NF4 weight read (34.6 MB), A and B read (1 MB each), the bf16 weight "
                  "written (134 MB).  Every tile reads its A slab (16 KB) and, at each new row of tiles, its B "
                  "rows from L2; each of the eight XCDs has an L2 of its own."]
        if wl == DECODE_ROT:
            L += ["", "The 192 calls rotate over 64 copies of the weight (551 MB of NF4), so every call's weight "
                  "comes from HBM."]
        write(os.path.join(PROFILES, f"hbm_traffic_{wl}.md"), L)


# --------------------------------------------------------------- counters --

CNAMES = [("fwd_rich", "fwd_rich (k_fwd8<256,1>)"), ("dx", "dx (k_dx8<256>)"),
          ("lora_proj_T", "lora_proj T = X A^T"), ("lora_proj_U", "lora_proj U = dY B"),
          ("token_reduce", "token_reduce dA, dB")]


def cmd_counters(a) -> None:
    n = 4096
    flops = {"fwd_rich": 2 * n ** 3 + 2 * n * n * 16, "dx": 2 * n ** 3 + 2 * n * n * 16,
             "lora_proj_T": 2 * n * n * 16, "lora_proj_U": 2 * n * n * 16, "token_reduce": 4 * n * n * 16}
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for d in a.dirs:
        seen = set()
        for r in csv.DictReader(open(find(d, "*counter_collection.csv"))):
            s = short_name(r["Kernel_Name"])
            if s not in flops:
                continue
            vals[s][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if (d, r["Dispatch_Id"]) not in seen:
                seen.add((d, r["Dispatch_Id"]))
                dur[s].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)

    def v(s, c):
        return statistics.mean(vals[s][c])

    simds, cus, peak = 1024, 256, 2516.6e12
    L = [f"# MFMA and instruction counters: QLoRA linear step, d = k = 4096, M = 4096, r = 16", "",
         "Three rocprofv3 counter passes over the training step (3 steps each; every figure is the mean over the "
         "kernel's dispatches), then `profile_summary.py counters --dirs gpurun_out/pmcA gpurun_out/pmcB "
         "gpurun_out/pmcC`:", "", "```"]
    for d, c in COUNTER_PASSES.items():
        L.append(PROFILE_CMD.format(t=120, c=c, d=d, args=COUNTER_ARGS))
    L += ["```", "",
          "Derived figures.  MFMA-busy cycles per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs (the counter equals "
          "flops / 1024 here: one bf16 MFMA SIMD-cycle per 1024 flops).  Shader clock = SQ_BUSY_CU_CYCLES / 256 CUs / "
          "duration.  MFMA busy = MFMA-busy cycles per SIMD / (clock x duration).  Against peak = flops / duration / "
          "2516.6 TFLOP/s (2.4 GHz).  Co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (MFMA cycles in "
          "which the SIMD also issued VALU work).  Durations are the counter runs' own dispatch times.", "",
          "| kernel | us | flops / MOPS_BF16 | clock GHz | MFMA busy | against 2.4 GHz peak | VALU / MFMA | "
          "LDS / MFMA | SALU / MFMA | co-issue | LDS command FIFO full |",
          "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for s, nm in CNAMES:
        if s not in dur:
            continue
        t = statistics.mean(dur[s])
        busy = v(s, "SQ_VALU_MFMA_BUSY_CYCLES") / simds
        clk = v(s, "SQ_BUSY_CU_CYCLES") / cus / t
        mf = v(s, "SQ_INSTS_MFMA")
        L.append(f"| {nm} | {t * 1e6:.1f} | {flops[s] / v(s, 'SQ_INSTS_VALU_MFMA_MOPS_BF16'):.0f} | {clk / 1e9:.2f} | "
                 f"{busy / (clk * t):.1%} | {flops[s] / t / peak:.1%} | {v(s, 'SQ_INSTS_VALU') / mf:.2f} | "
                 f"{v(s, 'SQ_INSTS_LDS') / mf:.2f} | {v(s, 'SQ_INSTS_SALU') / mf:.2f} | "
                 f"{v(s, 'SQ_VALU_MFMA_COEXEC_CYCLES') / v(s, 'SQ_VALU_MFMA_BUSY_CYCLES'):.1%} | "
                 f"{v(s, 'SQ_LDS_CMD_FIFO_FULL') / v(s, 'SQ_BUSY_CU_CYCLES'):.1%} |")
    L += ["", "Raw counter means per dispatch:", "", "| kernel | counter | value |", "|---|---|---:|"]
    for s, nm in CNAMES:
        for c in sorted(vals[s]):
            L.append(f"| {nm} | {c} | {v(s, c):.4g} |")
    write(os.path.join(PROFILES, f"mfma_counters_{TRAIN}.md"), L)


# --------------------------------------------------------- decode counters --

DECODE_COUNTERS = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_INSTS_VALU "
                   "SQ_INSTS_VMEM_RD SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def cmd_decode_counters(a) -> None:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(find(a.dir, "*counter_collection.csv"))):
        s = short_name(r["Kernel_Name"])
        if s not in ("fwd_decode", "fwd_decode_finish"):
            continue
        key = (s, symbol(r["Kernel_Name"]))
        vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    cmd = PROFILE_CMD.format(t=120, c=DECODE_COUNTERS, d="pmc_decode", args="--what decode_rot --steps 3")
    L = ["# Decode-call counters: forward at M = 16, d = k = 4096, r = 16, 64 rotating weight copies", "",
         "One rocprofv3 counter pass over 192 decode calls (three passes over 64 copies of the weight, so every "
         "call reads its weight from HBM), then `profile_summary.py decode-counters --dir gpurun_out/pmc_decode`:",
         "", "```", cmd, "```", "",
         "Per kernel, the mean over its dispatches.  Wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES (the share of the "
         "waves' lifetime spent waiting on an outstanding memory or LDS operation); instruction counts are per "
         "wave.  Durations are the counter run's own dispatch times (the counters serialise the dispatches).", "",
         "| kernel | dispatches | us | waves | VALU / wave | VMEM loads / wave | LDS / wave | wait share | "
         "dependency-wait share |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (s, sym), c in sorted(vals.items()):
        m = {n: statistics.mean(v) for n, v in c.items()}
        w = m["SQ_WAVES"]
        L.append(f"| {sym} | {len(dur[(s, sym)])} | {statistics.mean(dur[(s, sym)].values()):.2f} | {w:.0f} | "
                 f"{m['SQ_INSTS_VALU'] / w:.0f} | {m['SQ_INSTS_VMEM_RD'] / w:.1f} | {m['SQ_INSTS_LDS'] / w:.1f} | "
                 f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1%} | {m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1%} |")
    L += ["", "Raw counter means per dispatch:", "", "| kernel | counter | value |", "|---|---|---:|"]
    for (s, sym), c in sorted(vals.items()):
        for n in sorted(c):
            L.append(f"| {sym} | {n} | {statistics.mean(c[n]):.4g} |")
    write(os.path.join(PROFILES, f"decode_counters_{DECODE_ROT}.md"), L)


# ------------------------------------------------------------ L1 fetches --

FETCH_COUNTERS = ("TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum TCC_HIT_sum "
                  "TCC_MISS_sum SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE")
# Bytes one work-group must read (each runs on a CU of its own: one round of
# 256 work-groups), by kernel symbol prefix, for the workloads of
# profile_run.py: the 4096^2 training step (M = 4096, r = 16) and the
# M = 16 decode call (r = 16).
CU_READ_BYTES = {
    "k_fwd_dec1s<1, true, 4>": ("X 16 x 4096 + A 16 x 4096 (bf16) + codes of 16 rows", 2 * 16 * 4096 * 2 + 16 * 2048),
    "k_fwd_dec1<1, true>": ("X 16 x 4096 + A 16 x 4096 (bf16) + codes of 16 rows", 2 * 16 * 4096 * 2 + 16 * 2048),
    "k_proj<1, false>": ("X 16 rows + all of A (16 x 4096)", 16 * 4096 * 2 + 16 * 4096 * 2),
    "k_proj<1, true>": ("dY 16 rows + all of B (4096 x 16)", 16 * 4096 * 2 + 4096 * 16 * 2),
    "k_tokred<1, 3, 2>": ("a 32-column strip of X or dY over 4096 tokens + all of U or T", 4096 * 64 + 16 * 4096 * 2),
    "k_fwd8<256, 1>": ("X panel 256 x 4096 + codes of 256 rows", 256 * 4096 * 2 + 256 * 2048),
    "k_dx8<256, false>": ("dY panel 256 x 4096 + codes of a 256-column strip", 256 * 4096 * 2 + 4096 * 128),
}


def cmd_fetch(a) -> None:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(find(a.dir, "*counter_collection.csv"))):
        sym = symbol(r["Kernel_Name"])
        if sym not in CU_READ_BYTES:
            continue
        vals[sym][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[sym][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    cus = 256
    cmd = PROFILE_CMD.format(t=120, c=FETCH_COUNTERS, d="pmc_fetch", args="--what train,decode_rot --steps 3")
    L = ["# Vector L1 -> L2 read requests: training step (d = k = 4096, M = 4096, r = 16) and decode call "
         "(M = 16, r = 16, 64 rotating weight copies)", "",
         "One rocprofv3 counter pass, then `profile_summary.py fetch --dir gpurun_out/pmc_fetch`:", "",
         "```", cmd, "```", "",
         "Per kernel, the mean over its dispatches.  Requests per CU = TCP_TCC_READ_REQ_sum / 256.  Latency = "
         "TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (shader cycles from a CU's request to L2 until its "
         "data returns).  Clock = SQ_BUSY_CU_CYCLES / 256 / duration.  In flight per CU = "
         "TCP_TCC_READ_REQ_LATENCY_sum / 256 / (clock x duration): the mean number of a CU's read requests "
         "outstanding over the dispatch (Little's law).  Read bytes per CU: what one work-group must read (one "
         "work-group per CU), and that divided by the duration.", "",
         "| kernel | us | read bytes per CU | per CU GB/s | requests per CU | bytes / request | L2 hit | latency "
         "cycles (ns) | in flight per CU | clock GHz |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for sym in CU_READ_BYTES:
        if sym not in vals:
            continue
        m = {n: statistics.mean(v) for n, v in vals[sym].items()}
        t = statistics.mean(dur[sym].values())
        req = m["TCP_TCC_READ_REQ_sum"]
        lat = m["TCP_TCC_READ_REQ_LATENCY_sum"] / req
        clk = m["SQ_BUSY_CU_CYCLES"] / cus / t
        infl = m["TCP_TCC_READ_REQ_LATENCY_sum"] / cus / (clk * t)
        what, nbytes = CU_READ_BYTES[sym]
        hit = m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])
        L.append(f"| {sym} | {t * 1e6:.2f} | {nbytes / 1024:.0f} KB ({what}) | {nbytes / t / 1e9:.1f} | "
                 f"{req / cus:.0f} | {nbytes * cus / req:.0f} | {hit:.1%} | {lat:.0f} ({lat / clk * 1e9:.0f}) | "
                 f"{infl:.0f} | {clk / 1e9:.2f} |")
    L += ["", "Raw counter means per dispatch:", "", "| kernel | counter | value |", "|---|---|---:|"]
    for sym in CU_READ_BYTES:
        for n in sorted(vals.get(sym, {})):
            L.append(f"| {sym} | {n} | {statistics.mean(vals[sym][n]):.4g} |")
    write(os.path.join(PROFILES, "l1_fetch_counters.md"), L)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--bench-log", default=None, help="stdout of the profiled bench.py run (its JSON line)")
    f = sub.add_parser("traffic")
    f.add_argument("--fetch-dir", required=True)
    f.add_argument("--write-dir", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--dirs", nargs=3, required=True)
    dc = sub.add_parser("decode-counters")
    dc.add_argument("--dir", required=True)
    fe = sub.add_parser("fetch")
    fe.add_argument("--dir", required=True)
    a = ap.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters,
     "decode-counters": cmd_decode_counters, "fetch": cmd_fetch}[a.cmd](a)


if __name__ == "__main__":
    main()
