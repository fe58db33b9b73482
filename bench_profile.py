"""Summaries of rocprofv3 output for the bench workloads, written to profiles/.

    python bench_profile.py stats    <trace_dir> <workload> "<command>"
    python bench_profile.py traffic  <fetch_dir> <write_dir> <req_dir> <workload>
                                     "<fetch cmd>" "<write cmd>" "<req cmd>"
    python bench_profile.py counters <sq1_dir> <sq2_dir> <workload> "<cmd 1>" "<cmd 2>"
    python bench_profile.py l2       <l2_dir> <workload> "<command>"

`stats` reads <trace_dir>/run_kernel_stats.csv (rocprofv3 --kernel-trace
--stats -f csv -o run) and writes profiles/kernels_<workload>_stats.md.

`traffic` reads the counter_collection CSVs of three `rocprofv3 --pmc` runs of
`bench.py --copy-calibration`: FETCH_SIZE, WRITE_SIZE, and the TCC read
request counts by size (TCC_EA0_RDREQ{,_32B,_64B,_128B}_sum).  FETCH_SIZE and
WRITE_SIZE are scaled by what they read for the calibration copy, whose bytes
are known (bench.COPY_BYTES read and written); the request sizes give the
read bytes a second way, as a check of that scale on the kernel's own request
mix.  The per-dispatch figures of the workload's dominant kernel go to
profiles/<kernel>_<workload>_traffic.md with the hash of its sources.

`l2` reads one counter run of the L1-to-L2 and L2 request counters
(TCP_TCC_READ_REQ, TCP_TCC_WRITE_REQ, TCC_REQ, TCC_HIT, TCC_MISS, each summed
over the chip) of `bench.py --copy-calibration` and writes, per kernel, the
requests per launch and the L1-to-L2 read bytes they stand for (scaled by the
calibration copy's bytes per read request) against the kernel's algorithmic
read bytes, to profiles/<kernel>_<workload>_l2.md.

`counters` reads two SQ counter runs and writes, per kernel, the instruction
mix per wave, the VALU and MFMA busy fractions, the share of wave time spent
waiting, and the LDS bank-conflict cycles, to
profiles/<kernel>_<workload>_counters.md.
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
           "route_large_kernel": "route", "attend_kernel": "attend", "image_kernel": "image",
           "small_kernel": "small", "kv_pool_kernel": "kv_pool",
           "lepe_table_kernel": "lepe_table"}
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


def write_traffic(fetch_dir: str, write_dir: str, req_dir: str, workload: str, fetch_cmd: str,
                  write_cmd: str, req_cmd: str) -> str:
    from vision_transformer_sparse_region_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    kernel = bench.kernel_name(wl)
    fetch, nf = counter_means(fetch_dir, "FETCH_SIZE")
    write, nw = counter_means(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the calibration copy kernel is missing from the counter runs")
    f_fetch = bench.COPY_BYTES / (fetch["copy"] * 1024)
    f_write = bench.COPY_BYTES / (write["copy"] * 1024)
    # read requests by size: bytes = 32 n32 + 64 n64 + 128 n128
    req = {c: counter_means(req_dir, f"TCC_EA0_RDREQ{c}_sum")[0]
           for c in ("", "_32B", "_64B", "_128B")}

    def req_bytes(k):
        return 32 * req["_32B"].get(k, 0) + 64 * req["_64B"].get(k, 0) + \
            128 * req["_128B"].get(k, 0)
    f_req = bench.COPY_BYTES / req_bytes("copy") if req_bytes("copy") else None
    alg = bench.algorithmic_bytes(wl)
    per = {}
    for k in fetch:
        if k == "copy" or k not in write:
            continue
        rd, wr = fetch[k] * 1024 * f_fetch, write[k] * 1024 * f_write
        per[k] = {"fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
                  "read_bytes": rd, "write_bytes": wr, "hbm_bytes": rd + wr,
                  "rdreq": req[""].get(k), "rdreq_32b": req["_32B"].get(k),
                  "rdreq_64b": req["_64B"].get(k), "rdreq_128b": req["_128B"].get(k),
                  "read_bytes_by_request_size": req_bytes(k) * f_req if f_req else None,
                  "dispatches": min(nf.get(k, 0), nw.get(k, 0))}
    rec = {
        "workload": workload,
        "kernel": kernel,
        "kernel_source_sha256_16": bench.kernel_source_hash(kernel),
        "hbm_bytes_per_launch": per[kernel]["hbm_bytes"],
        "algorithmic_bytes_per_launch": alg["attend"],
        "copy_bytes": bench.COPY_BYTES,
        "copy_fetch_kib_raw": fetch["copy"], "copy_write_kib_raw": write["copy"],
        "copy_rdreq": {c or "all": req[c].get("copy") for c in req},
        "fetch_scale": f_fetch, "write_scale": f_write, "request_scale": f_req,
        "kernels": per,
    }
    lines = [f"# HBM traffic per launch, workload `{workload}`, kernel `{kernel}`", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from rocprofv3 counter runs, each",
             f"scaled by the same counter's reading for a {bench.COPY_BYTES >> 20} MiB device copy "
             "(bytes known: read once, written once).  The read bytes again from the TCC read",
             "requests by size (32, 64, 128 bytes), scaled the same way, check that scale on each",
             "kernel's own request mix.", "",
             "Commands (from the repository root):", "", "```", fetch_cmd, write_cmd, req_cmd,
             "```", "",
             "| kernel | FETCH KiB raw | WRITE KiB raw | read MB | write MB | total MB | "
             "read MB by request size |",
             "|---|---|---|---|---|---|---|"]
    for k, v in per.items():
        rq = v["read_bytes_by_request_size"]
        lines.append(f"| {k} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | "
                     f"{v['read_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} | "
                     f"{v['hbm_bytes'] / 1e6:.2f} | "
                     f"{rq / 1e6 if rq is not None else float('nan'):.2f} |")
    lines += ["", f"Copy calibration: FETCH {fetch['copy']:.0f} KiB, WRITE {write['copy']:.0f} KiB "
              f"for {bench.COPY_BYTES >> 10} KiB each way; scale {f_fetch:.4f} (fetch), "
              f"{f_write:.4f} (write), {f_req if f_req else float('nan'):.4f} (read requests).",
              "", f"Algorithmic bytes of `{kernel}` per launch: {alg['attend'] / 1e6:.2f} MB.",
              "", "```json", json.dumps(rec, indent=1), "```", ""]
    out = bench.traffic_summary_path(workload, kernel)
    os.makedirs(bench.PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    return out


SQ_COUNTERS = ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VMEM_RD",
               "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32",
               "GRBM_GUI_ACTIVE")
CUS, SIMDS, XCDS = 256, 1024, 8


def write_counters(sq1_dir: str, sq2_dir: str, workload: str, cmd1: str, cmd2: str) -> str:
    from vision_transformer_sparse_region_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    kernel = bench.kernel_name(wl)
    vals = defaultdict(dict)
    for d in (sq1_dir, sq2_dir):
        for c in SQ_COUNTERS:
            means, _ = counter_means(d, c)
            for k, v in means.items():
                if k != "copy":
                    vals[k].setdefault(c, v)
    rows = []
    for k, c in vals.items():
        waves = c.get("SQ_WAVES") or 1.0
        # GRBM_GUI_ACTIVE is summed over the XCDs: per XCD, the kernel's cycles
        cyc = (c.get("GRBM_GUI_ACTIVE") or 0.0) / XCDS
        rows.append({
            "kernel": k, "waves": waves,
            "valu_per_wave": c.get("SQ_INSTS_VALU", 0) / waves,
            "mfma_per_wave": c.get("SQ_INSTS_MFMA", 0) / waves,
            "lds_per_wave": c.get("SQ_INSTS_LDS", 0) / waves,
            "vmem_rd_per_wave": c.get("SQ_INSTS_VMEM_RD", 0) / waves,
            "trans_per_wave": c.get("SQ_INSTS_VALU_TRANS_F32", 0) / waves,
            "valu_busy_pct": 100 * c.get("SQ_ACTIVE_INST_VALU", 0) / (CUS * cyc) if cyc else None,
            "mfma_busy_pct": 100 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (SIMDS * cyc)
            if cyc else None,
            "wait_inst_share": c.get("SQ_WAIT_INST_ANY", 0) / c["SQ_WAVE_CYCLES"]
            if c.get("SQ_WAVE_CYCLES") else None,
            "lds_conflict_per_active": c.get("SQ_LDS_BANK_CONFLICT", 0) / c["SQ_ACTIVE_INST_LDS"]
            if c.get("SQ_ACTIVE_INST_LDS") else None,
            "gui_active_cycles_per_xcd": cyc,
            "raw": c,
        })
    fmt = lambda x, f="{:.1f}": "-" if x is None else f.format(x)
    lines = [f"# SQ counters per dispatch, workload `{workload}` (dominant kernel `{kernel}`)", "",
             "Two rocprofv3 counter runs (8 SQ counters and GRBM_GUI_ACTIVE each), averaged per",
             "dispatch.  VALU busy = SQ_ACTIVE_INST_VALU / (CUs x GRBM cycles per XCD) and MFMA",
             "busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM cycles per XCD), rocprofv3's VALUBusy",
             "and MfmaUtil; wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waves stalled on a",
             "dependency); LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS.", "",
             "Commands (from the repository root):", "", "```", cmd1, cmd2, "```", "",
             "| kernel | waves | VALU/wave | MFMA/wave | LDS/wave | VMEM rd/wave | exp/wave | "
             "VALU busy % | MFMA busy % | wait share | LDS conflict/active |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['kernel']} | {r['waves']:.0f} | {r['valu_per_wave']:.0f} | "
                     f"{r['mfma_per_wave']:.0f} | {r['lds_per_wave']:.0f} | "
                     f"{r['vmem_rd_per_wave']:.0f} | {r['trans_per_wave']:.0f} | "
                     f"{fmt(r['valu_busy_pct'])} | {fmt(r['mfma_busy_pct'])} | "
                     f"{fmt(r['wait_inst_share'], '{:.2f}')} | "
                     f"{fmt(r['lds_conflict_per_active'], '{:.2f}')} |")
    lines += ["", "```json", json.dumps({"workload": workload, "kernel": kernel,
                                         "kernel_source_sha256_16": bench.kernel_source_hash(kernel),
                                         "kernels": rows}, indent=1), "```", ""]
    out = os.path.join(bench.PROFILES, f"{kernel}_{workload}_counters.md")
    os.makedirs(bench.PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    return out


L2_COUNTERS = ("TCP_TCC_READ_REQ_sum", "TCP_TCC_WRITE_REQ_sum", "TCC_REQ_sum", "TCC_HIT_sum",
               "TCC_MISS_sum")


def write_l2(l2_dir: str, workload: str, command: str) -> str:
    from vision_transformer_sparse_region_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    kernel = bench.kernel_name(wl)
    vals = {c: counter_means(l2_dir, c)[0] for c in L2_COUNTERS}
    rd = vals["TCP_TCC_READ_REQ_sum"]
    if "copy" not in rd:
        raise SystemExit("the calibration copy kernel is missing from the counter run")
    # the copy reads COPY_BYTES once: bytes per L1-to-L2 read request
    bpr = bench.COPY_BYTES / rd["copy"]
    alg = bench.algorithmic_bytes(wl)["attend"]
    # algorithmic reads: the kernel's bytes less its output (S) and routing ids (I)
    out_bytes = wl.tokens * wl.channels * (2 if wl.dtype == "bf16" else 4)
    ids = wl.batch * wl.num_heads * wl.regions * wl.topk_effective * 4
    alg_read = alg - out_bytes - ids
    per = {}
    for k in rd:
        if k == "copy":
            continue
        per[k] = {c: vals[c].get(k) for c in L2_COUNTERS}
        # a request moves 64 or 128 bytes (the copy's are all 128): the two
        # bounds of the bytes behind a kernel's requests
        per[k]["l1_to_l2_read_bytes"] = rd[k] * bpr
        per[k]["l1_to_l2_read_bytes_at_64"] = rd[k] * 64
    rec = {"workload": workload, "kernel": kernel,
           "kernel_source_sha256_16": bench.kernel_source_hash(kernel),
           "copy_bytes": bench.COPY_BYTES, "copy_read_requests": rd["copy"],
           "bytes_per_read_request": bpr, "algorithmic_read_bytes": alg_read,
           "l2_read_amplification": per[kernel]["l1_to_l2_read_bytes"] / alg_read,
           "l2_read_amplification_at_64": per[kernel]["l1_to_l2_read_bytes_at_64"] / alg_read,
           "kernels": per}
    lines = [f"# L2 requests per launch, workload `{workload}`, kernel `{kernel}`", "",
             "L1-to-L2 read and write requests (TCP_TCC_*_REQ) and L2 requests, hits and misses",
             "(TCC_*), summed over the chip, per dispatch.  A read request moves 64 or 128 bytes;",
             f"the calibration copy's are all {bpr:.0f} bytes (it reads {bench.COPY_BYTES >> 20} MiB once).  The read bytes",
             "are given at 128 bytes a request (an upper bound) and at 64 (a lower bound); the",
             "amplification is those bytes over the kernel's algorithmic reads (its compulsory",
             "bytes less the output and the routing ids): the bytes its CUs pull from L2 for",
             "each byte the method must read.", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "| kernel | L1-to-L2 read req | write req | L2 req | L2 hit | L2 miss | "
             "L1-to-L2 read MB (128 / 64 B a request) |",
             "|---|---|---|---|---|---|---|"]
    for k, v in per.items():
        lines.append(f"| {k} | {v['TCP_TCC_READ_REQ_sum'] or 0:.0f} | "
                     f"{v['TCP_TCC_WRITE_REQ_sum'] or 0:.0f} | {v['TCC_REQ_sum'] or 0:.0f} | "
                     f"{v['TCC_HIT_sum'] or 0:.0f} | {v['TCC_MISS_sum'] or 0:.0f} | "
                     f"{v['l1_to_l2_read_bytes'] / 1e6:.2f} / "
                     f"{v['l1_to_l2_read_bytes_at_64'] / 1e6:.2f} |")
    lines += ["", f"Copy calibration: {rd['copy']:.0f} read requests for "
              f"{bench.COPY_BYTES >> 20} MiB, {bpr:.1f} bytes a request.", "",
              f"`{kernel}`: {per[kernel]['l1_to_l2_read_bytes_at_64'] / 1e6:.2f} to "
              f"{per[kernel]['l1_to_l2_read_bytes'] / 1e6:.2f} MB from L2 against "
              f"{alg_read / 1e6:.2f} MB of algorithmic reads, "
              f"{rec['l2_read_amplification_at_64']:.2f}x to {rec['l2_read_amplification']:.2f}x.",
              "", "```json", json.dumps(rec, indent=1), "```", ""]
    out = os.path.join(bench.PROFILES, f"{kernel}_{workload}_l2.md")
    os.makedirs(bench.PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    return out


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        print(write_stats(argv[1], argv[2], argv[3]))
    elif len(argv) >= 8 and argv[0] == "traffic":
        print(write_traffic(*argv[1:8]))
    elif len(argv) >= 6 and argv[0] == "counters":
        print(write_counters(*argv[1:6]))
    elif len(argv) >= 4 and argv[0] == "l2":
        print(write_l2(*argv[1:4]))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
