"""Counter and trace summaries for the persistent kernel (rocprofv3 on MI355X).

Two entry points, both run from the repository root:

  python -m persistent_whole_step_amd.profiling run WORKLOAD [--launches N]
      The program to put under `rocprofv3 --pmc FETCH_SIZE` (then
      `--pmc WRITE_SIZE`): N launches of the workload's whole step on resident
      inputs, then one device-to-device copy of exactly COPY_BYTES, whose
      counter readings calibrate the counters (bytes the counter reports per
      byte a plain copy kernel moves).

  python -m persistent_whole_step_amd.profiling summarize WORKLOAD \\
          --fetch FETCH_CSV --write WRITE_CSV [--stats STATS_CSV] --command CMD ...
      Reads rocprofv3's counter_collection CSVs (and optionally the
      kernel_stats CSV of a `--kernel-trace --stats` run) and writes
      profiles/tk_persistent_<workload>_traffic.json and a short text summary.

The counters are summed over all instances and reported in KiB per dispatch;
the calibration turns them into bytes.  The summary records the hash of the
kernel sources it was taken on: bench.py reports traffic only while the
sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written
KERNEL = "tk_persistent"


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def cmd_run(args):
    import torch
    bench = _bench()
    # the bench's launch configuration: an ordinary launch of the co-resident
    # grid (cooperative launches make the profiler crash in its exit handlers)
    r = bench.Runner(args.workload, launch_mode=1)
    for i in range(args.launches):
        r.step(i)
    torch.cuda.synchronize()
    r.check_not_aborted()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    # Release every device resource here, while the runtime is whole: a
    # device call made from a finaliser after the profiler's tool has shut
    # down at exit crashes the process.
    r.close()
    del src, dst, r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"[profiling] {args.workload}: {args.launches} launches, copy of {COPY_BYTES} bytes", flush=True)


def _counter_rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter, match):
    """Mean over dispatches of a kernel (name contains `match`) of the counter
    summed over instances."""
    per = defaultdict(float)
    for r in rows:
        if r.get("Counter_Name") != counter or match not in r.get("Kernel_Name", ""):
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)


def _copy_kernel_reading(rows, counter):
    """Largest single dispatch reading among the runtime's copy kernels: the
    calibration copy moves far more bytes than any other copy of the run."""
    per = defaultdict(float)
    names = {}
    for r in rows:
        if r.get("Counter_Name") != counter or "copy" not in r.get("Kernel_Name", "").lower():
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    if not per:
        return None, None
    d = max(per, key=per.get)
    return per[d], names[d]


def cmd_summarize(args):
    bench = _bench()
    name = bench.WORKLOAD_NAMES[args.workload]
    fetch_rows = _counter_rows(args.fetch)
    write_rows = _counter_rows(args.write)
    fetch_kib, nf = _per_dispatch(fetch_rows, "FETCH_SIZE", KERNEL)
    write_kib, nw = _per_dispatch(write_rows, "WRITE_SIZE", KERNEL)
    copy_fetch, copy_name_f = _copy_kernel_reading(fetch_rows, "FETCH_SIZE")
    copy_write, copy_name_w = _copy_kernel_reading(write_rows, "WRITE_SIZE")
    if None in (fetch_kib, write_kib, copy_fetch, copy_write):
        raise SystemExit("profiling: missing counter rows (kernel or calibration copy)")
    # bytes moved per counter unit, from the copy of known size
    f_scale = COPY_BYTES / copy_fetch
    w_scale = COPY_BYTES / copy_write
    fetch_b = fetch_kib * f_scale
    write_b = write_kib * w_scale
    out = {
        "kernel": KERNEL,
        "workload": name,
        "source_hash": bench.source_hash(),
        "dispatches": {"fetch": nf, "write": nw},
        "FETCH_SIZE_kib_per_dispatch": round(fetch_kib, 1),
        "WRITE_SIZE_kib_per_dispatch": round(write_kib, 1),
        "calibration": {"copy_bytes": COPY_BYTES, "copy_kernel": [copy_name_f, copy_name_w],
                        "FETCH_SIZE_kib": round(copy_fetch, 1), "WRITE_SIZE_kib": round(copy_write, 1),
                        "bytes_per_fetch_unit": round(f_scale, 3), "bytes_per_write_unit": round(w_scale, 3)},
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(fetch_b + write_b),
        "commands": args.command,
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", f"{KERNEL}_{name}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"[profiling] wrote {path}")
    if args.stats:
        with open(args.stats, newline="") as f:
            rows = list(csv.DictReader(f))
        lines = [f"# {KERNEL} on {name}: rocprofv3 kernel statistics", "",
                 "Command (from the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp):", ""]
        lines += [f"    {c}" for c in args.stats_command]
        lines += ["", "| kernel | calls | total ns | average ns | min ns | max ns | % |",
                  "|---|---|---|---|---|---|---|"]
        for r in rows:
            nm = r.get("Name", r.get("KernelName", "?"))
            short = nm if len(nm) <= 60 else nm[:57] + "..."
            lines.append(f"| {short} | {r.get('Calls')} | {r.get('TotalDurationNs')} | {r.get('AverageNs')} | "
                         f"{r.get('MinNs')} | {r.get('MaxNs')} | {r.get('Percentage')} |")
        lines += ["", f"HBM traffic per launch (counters scaled by the {COPY_BYTES}-byte copy calibration): "
                      f"fetch {int(fetch_b)} B, write {int(write_b)} B "
                      f"(FETCH_SIZE {fetch_kib:.1f} KiB x {f_scale:.1f}, WRITE_SIZE {write_kib:.1f} KiB x {w_scale:.1f}).",
                  f"Source hash {out['source_hash']}."]
        spath = os.path.join(ROOT, "profiles", f"{KERNEL}_{name}_kernel_stats.md")
        with open(spath, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"[profiling] wrote {spath}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("run")
    a.add_argument("workload")
    a.add_argument("--launches", type=int, default=20)
    b = sub.add_parser("summarize")
    b.add_argument("workload")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--stats")
    b.add_argument("--command", action="append", default=[], help="counter commands, for the record")
    b.add_argument("--stats-command", action="append", default=[], help="kernel-trace command, for the record")
    args = ap.parse_args()
    if args.cmd == "run":
        cmd_run(args)
    else:
        cmd_summarize(args)


if __name__ == "__main__":
    main()
