"""Summaries of rocprofv3 output for the bench workloads, written to profiles/.

    python bench_profile.py stats   <trace_dir> <workload> "<command>"
    python bench_profile.py traffic <fetch_dir> <write_dir> <workload> "<fetch cmd>" "<write cmd>"

`stats` reads <trace_dir>/run_kernel_stats.csv (rocprofv3 --kernel-trace
--stats -f csv -o run) and writes profiles/kernels_<workload>_stats.md.

`traffic` reads the counter_collection CSVs of two `rocprofv3 --pmc` runs of
`bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE).  Each counter is
scaled by what it reads for the calibration copy, whose bytes are known
(bench.COPY_BYTES read and written), and the per-dispatch averages of the
attention kernel go to profiles/attend_<workload>_traffic.md together with
the hash of the kernel sources they were taken on.
"""
from __future__ import annotations

import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

KERNELS = {"pool_qk_kernel": "region_pool", "pool_route_kernel": "region_pool_and_route",
           "proj_qkv_kernel": "qkv_projection",
           "proj_out_kernel": "output_projection", "route_small_kernel": "route",
           "route_large_kernel": "route", "attend_kernel": "attend"}
COPY_KERNELS = ("__amd_rocclr_copyBuffer",)


def short_name(full: str):
    for key, short in KERNELS.items():
        if key in full:
            return short
    for key in COPY_KERNELS:
        if key in full:
            return "copy"
    return None


def write_stats(trace_dir: str, workload: str, command: str) -> str:
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    out = os.path.join(bench.PROFILES, f"kernels_{workload}_stats.md")
    lines = [f"# Kernel durations, workload `{workload}`", "",
             "rocprofv3 kernel-trace statistics (all dispatches of the run, warm-up included).", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = short_name(r["Name"]) or r["Name"][:60]
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    lines += ["", "Full kernel names:", ""]
    lines += [f"- `{r['Name']}`" for r in rows]
    os.makedirs(bench.PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def counter_means(run_dir: str, counter: str):
    """Average value of `counter` per dispatch, by short kernel name.  For the
    copy kernel only the calibration copies count: the last
    bench.COPY_REPS copy dispatches (earlier ones are host-to-device uploads)."""
    vals = defaultdict(list)
    rows = list(csv.DictReader(open(os.path.join(run_dir, "run_counter_collection.csv"))))
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        name = short_name(r["Kernel_Name"])
        if name:
            vals[name].append(float(r["Counter_Value"]))
    if "copy" in vals:
        vals["copy"] = vals["copy"][-bench.COPY_REPS:]
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def write_traffic(fetch_dir: str, write_dir: str, workload: str, fetch_cmd: str,
                  write_cmd: str) -> str:
    fetch, nf = counter_means(fetch_dir, "FETCH_SIZE")
    write, nw = counter_means(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the calibration copy kernel is missing from the counter runs")
    f_fetch = bench.COPY_BYTES / (fetch["copy"] * 1024)
    f_write = bench.COPY_BYTES / (write["copy"] * 1024)
    from vision_transformer_sparse_region_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    alg = bench.algorithmic_bytes(wl)
    per = {}
    for k in ("region_pool", "route", "attend"):
        if k in fetch and k in write:
            rd, wr = fetch[k] * 1024 * f_fetch, write[k] * 1024 * f_write
            per[k] = {"fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
                      "read_bytes": rd, "write_bytes": wr, "hbm_bytes": rd + wr,
                      "dispatches": min(nf.get(k, 0), nw.get(k, 0))}
    rec = {
        "workload": workload,
        "kernel": "attend",
        "kernel_source_sha256_16": bench.kernel_source_hash(),
        "hbm_bytes_per_launch": per["attend"]["hbm_bytes"],
        "algorithmic_bytes_per_launch": alg["attend"],
        "copy_bytes": bench.COPY_BYTES,
        "copy_fetch_kib_raw": fetch["copy"], "copy_write_kib_raw": write["copy"],
        "fetch_scale": f_fetch, "write_scale": f_write,
        "kernels": per,
    }
    lines = [f"# HBM traffic per launch, workload `{workload}`", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 counter runs, each",
             f"scaled by the same counter's reading for a {bench.COPY_BYTES >> 20} MiB device copy "
             "(bytes known: read once, written once).", "",
             "Commands (from the repository root):", "", "```", fetch_cmd, write_cmd, "```", "",
             "| kernel | FETCH KiB raw | WRITE KiB raw | read MB | write MB | total MB |",
             "|---|---|---|---|---|---|"]
    for k, v in per.items():
        lines.append(f"| {k} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | "
                     f"{v['read_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} | "
                     f"{v['hbm_bytes'] / 1e6:.2f} |")
    lines += ["", f"Copy calibration: FETCH {fetch['copy']:.0f} KiB, WRITE {write['copy']:.0f} KiB "
              f"for {bench.COPY_BYTES >> 10} KiB each way; scale {f_fetch:.4f} (fetch), "
              f"{f_write:.4f} (write).", "",
              f"Algorithmic bytes of the attention kernel per launch: {alg['attend'] / 1e6:.2f} MB.",
              "", "```json", json.dumps(rec, indent=1), "```", ""]
    out = bench.traffic_summary_path(workload)
    os.makedirs(bench.PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    return out


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        print(write_stats(argv[1], argv[2], argv[3]))
    elif len(argv) >= 6 and argv[0] == "traffic":
        print(write_traffic(argv[1], argv[2], argv[3], argv[4], argv[5]))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
