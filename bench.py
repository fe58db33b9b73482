"""Benchmark of the BRA forward (libbra.so) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage1]

A step is one bra_forward (region-means kernel, routing kernel,
attention/LePE kernel) over one batch of the workload, inputs already in HBM.  By default
the steps rotate over enough input/output buffer sets that consecutive steps
never find their inputs in the 256 MB last-level cache (MALL), so the
figures are HBM figures.  Prints one JSON line with the throughput, the
roofline of the dominant kernel (timed per launch with HIP events inside the
timed region) and the CPU oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BRA fwd tokens/s (bf16) + % HBM roofline / % MFMA peak vs CPU oracle"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "vision_transformer_sparse_region_amd", "csrc")
# Sources that determine each dominant kernel's code (its counters go stale
# when any of them changes).
KERNEL_SOURCES = {
    "attend": ("bra_attend.hip", "bra_device.h", "bra_shapes.h", "bra_launch.h"),
    "image": ("bra_image.hip", "bra_image.h", "bra_device.h", "bra_launch.h"),
    "small": ("bra_small.hip", "bra_small.h", "bra_device.h", "bra_launch.h"),
}
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20  # size of the calibration copy (read and written once each)
COPY_REPS = 5
# the embedded workloads of the benchmark table: at least this many timed and
# untimed steps
CONFIG_MIN_STEPS = 200
CONFIG_MIN_WARMUP = 50


def _code_only(text: str) -> str:
    """Source text without comments and blank lines: an edit to a comment
    leaves the compiled kernel, and so the counters taken on it, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash(kernel: str = "attend") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def route_in_attend(wl, shared_routing: bool = False) -> bool:
    """Maps of at most 64 regions with at most 4 heads are routed inside the
    attention kernel (per-head routing)."""
    return wl.regions <= 64 and wl.num_heads <= 4 and not shared_routing


def route_in_pool(wl, shared_routing: bool = False) -> bool:
    """bf16 maps of at most 64 regions routed outside the attention kernel,
    with regions of at most 16 tokens and R * t <= 256: one kernel computes
    the region means and the routing."""
    return (wl.dtype == "bf16" and not shared_routing and wl.regions <= 64 and
            not route_in_attend(wl, shared_routing) and wl.tokens_per_region <= 16 and
            wl.regions * wl.tokens_per_region <= 256)


# (window side, n_win, heads, k) of the whole-image kernel's compiled shapes
IMAGE_SHAPES = {(4, 7, 4, 4), (2, 7, 8, 16)}


def image_path(wl, shared_routing: bool = False, kv_ratio: int = 1) -> bool:
    """bf16 maps whose head-group K and V fit LDS: one kernel runs the whole
    forward (means, routing, attention, LePE)."""
    hs, ws = wl.height // wl.n_win, wl.width // wl.n_win
    return (wl.dtype == "bf16" and not shared_routing and max(kv_ratio, 1) == 1 and hs == ws and
            (hs, wl.n_win, wl.num_heads, wl.topk_effective) in IMAGE_SHAPES)


def small_lds_bytes(wl) -> int:
    """LDS of the one-launch fp32 kernel (its layout: the head's K map, the
    fp64 K means, the routed V rows, the probabilities, the V window with its
    halo, the Q rows, the LePE weights, the ids and the token tables; the DMA
    arrays whole rounds of 256 16-byte slots)."""
    t, nk = wl.tokens_per_region, wl.topk_effective * wl.tokens_per_region
    hs, ws = wl.height // wl.n_win, wl.width // wl.n_win
    rnd = lambda slots: -(-slots // 256) * 4096
    a16 = lambda x: (x + 15) & ~15
    off = rnd(wl.height * wl.width * 8)
    off = a16(off + wl.regions * 32 * 8)
    off += rnd(nk * 8)
    off = a16(off + t * (nk + 4) * 4)
    off += rnd((hs + 4) * (ws + 4) * 8)
    off += rnd(t * 8)
    off = a16(off + (32 * 25 + 32) * 4)
    off = a16(off + 2 * 16 * 4)
    return a16(off + 2 * 64 * 4)


def small_path(wl, shared_routing: bool = False, kv_ratio: int = 1) -> bool:
    """fp32 problems of at most 256 (image, head, region) triples: one kernel,
    one workgroup per triple, runs the whole forward."""
    t = wl.tokens_per_region
    return (wl.dtype == "f32" and not shared_routing and max(kv_ratio, 1) == 1 and
            wl.batch * wl.num_heads * wl.regions <= 256 and wl.regions <= 64 and t <= 64 and
            wl.topk_effective <= 16 and small_lds_bytes(wl) <= 160 * 1024)


def one_kernel(wl, shared_routing: bool = False, kv_ratio: int = 1) -> bool:
    return image_path(wl, shared_routing, kv_ratio) or small_path(wl, shared_routing, kv_ratio)


def out_proj_in_attend(wl) -> bool:
    """The output projection runs in the attention kernel's epilogue when
    C <= 4 t, else as a kernel of its own over the attention output."""
    return wl.channels <= 4 * wl.tokens_per_region


def qmean_in_attend(wl, shared_routing: bool = False) -> bool:
    """bf16 maps routed inside the attention kernel whose query tiles fit the
    four waves' first jobs: the attention kernel sums the Q means itself and
    the pool kernel reads only K.  (The split of a region's 16-query tiles
    over the waves: at most 2 tiles per job, spare waves take extra groups.)"""
    if wl.dtype != "bf16" or not route_in_attend(wl, shared_routing):
        return False
    qt = (wl.tokens_per_region + 15) // 16
    spread = min(max(1, 4 // wl.num_heads), qt)
    groups = max(spread, (qt + 1) // 2)
    per_group = (qt + groups - 1) // groups
    return wl.num_heads * ((qt + per_group - 1) // per_group) <= 4


def kmean32(wl, shared_routing: bool = False) -> bool:
    """Mirrors the library: the routing inside the attention kernel screens
    with an fp32 copy of the K means (written next to the fp64 ones) when a
    window holds at least 32 tokens."""
    return route_in_attend(wl, shared_routing) and wl.tokens_per_region >= 32


def algorithmic_bytes(wl, shared_routing: bool = False, kv_ratio: int = 1,
                      projections: bool = False) -> dict:
    """Bytes each kernel must move once per launch (unique bytes; the k-fold
    re-reads of routed K/V, of the LePE halo and of the K means are cache
    traffic).  When the routing runs inside the attention kernel, that kernel
    also reads the means and writes the ids; when it also sums the Q means,
    only the K means are written and read.  Where it screens with fp32 K
    means, those are written besides the fp64 ones and read instead of them
    (the fp64 means are read only for near ties)."""
    es = 2 if wl.dtype == "bf16" else 4
    S = wl.tokens * wl.channels * es                     # one [B,H,W,C] tensor
    M = wl.batch * wl.channels * wl.regions * 8          # one fp64 [B,heads,R,32] mean array
    idx = wl.batch * (1 if shared_routing else wl.num_heads) * wl.regions * \
        wl.topk_effective * 4
    lepe = wl.channels * 26 * 4
    r2 = max(kv_ratio, 1) ** 2
    # with KV downsampling a pooling pass reads k and v and writes 2S/r^2; the
    # attention then gathers the pooled K/V (2S/r^2) and still reads v for LePE
    kvpool = 2 * S + 2 * S // r2 if r2 > 1 else 0
    attend = (3 * S + 2 * S // r2 if r2 > 1 else 4 * S) + idx + lepe
    k32 = M // 2 if kmean32(wl, shared_routing) else 0   # fp32 K means
    kread = k32 if k32 else M                            # K means the attention reads
    if one_kernel(wl, shared_routing, kv_ratio) and not projections:
        # one kernel: q, k, v read once, out written once, the ids exported
        return {"pool": 0, "route": 0, "attend": attend, "S": S}
    if projections:
        # the qkv projection reads x and the weights, writes q, k, v and both
        # means; the attention kernel also reads the output weights.  (When
        # the output projection is a kernel of its own, the attention slot
        # times both kernels; y's round trip between them is not counted.)
        wq, wo = 3 * wl.channels * wl.channels * es, wl.channels * wl.channels * es
        pool = S + wq + 3 * wl.channels * 4 + 3 * S + 2 * M + k32 + kvpool
        att = attend + wo + wl.channels * 4
        if image_path(wl, shared_routing, kv_ratio):
            return {"pool": pool, "route": 0, "attend": att, "S": S}
        if route_in_attend(wl, shared_routing):
            return {"pool": pool, "route": 0, "attend": att + M + kread, "S": S}
        return {"pool": pool, "route": 2 * M + idx, "attend": att, "S": S}
    if route_in_pool(wl, shared_routing):
        # one kernel reads q and k and writes the ids; no mean array in HBM
        return {"pool": 2 * S + idx + kvpool, "route": 0, "attend": attend, "S": S}
    if qmean_in_attend(wl, shared_routing):
        return {"pool": S + M + k32 + kvpool, "route": 0, "attend": attend + kread, "S": S}
    if route_in_attend(wl, shared_routing):
        return {"pool": 2 * S + 2 * M + k32 + kvpool, "route": 0, "attend": attend + M + kread,
                "S": S}
    return {
        "pool": 2 * S + 2 * M + kvpool,                  # read q, k; write both means
        "route": 2 * M + idx,                            # read both means; write the ids
        "attend": attend,                                # read q, k, v, ids, w; write out
        "S": S,
    }


def attention_flops(wl, kv_ratio: int = 1) -> float:
    return 4.0 * wl.tokens * wl.num_heads * wl.topk_effective * \
        (wl.tokens_per_region // max(kv_ratio, 1) ** 2) * wl.head_dim


def traffic_summary_path(workload: str, kernel: str = "attend") -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")


def read_traffic_record(path: str):
    """The JSON record inside the ```json fence of a traffic summary."""
    with open(path) as f:
        text = f.read()
    start = text.index("```json") + len("```json")
    return json.loads(text[start:text.index("```", start)])


def stored_traffic(workload: str, kernel: str = "attend"):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary, or None when absent or taken on a different
    kernel source."""
    path = traffic_summary_path(workload, kernel)
    if not os.path.exists(path):
        return None
    rec = read_traffic_record(path)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, inputs, gpu_out, target_s: float = 10.0, shared: bool = False,
                 kv_ratio: int = 1) -> dict:
    """Time the CPU oracle on the first images of the same batch (a bounded
    sample) and check the GPU output for those images against it."""
    import numpy as np

    import oracle

    def run(nimg):
        cfg = oracle.OracleConfig(nimg, wl.height, wl.width, wl.channels, wl.num_heads,
                                  wl.n_win, wl.topk)
        f = {n: inputs[n][:nimg].double().numpy() for n in ("q", "k", "v")}
        w, b = inputs["lepe_w"].double().numpy(), inputs["lepe_b"].double().numpy()
        t0 = time.perf_counter()
        if shared and kv_ratio > 1:
            idx = oracle.bra_forward_shared(cfg, f["q"], f["k"], f["v"])["idx"]
            full = np.ascontiguousarray(np.repeat(idx[:, None], wl.num_heads, axis=1))
            res = {"out": oracle.attend_kvds(cfg, kv_ratio, f["q"], f["k"], f["v"], full) +
                   oracle.lepe(cfg, f["v"], w, b)}
        elif kv_ratio > 1:
            res = oracle.bra_forward_kvds(cfg, kv_ratio, f["q"], f["k"], f["v"], w, b)
        elif shared:
            res = oracle.bra_forward_shared(cfg, f["q"], f["k"], f["v"], w, b)
        else:
            res = oracle.bra_forward(cfg, f["q"], f["k"], f["v"], w, b)
        return time.perf_counter() - t0, res

    dt, res = run(1)
    nimg = int(max(1, min(wl.batch, target_s / max(dt, 1e-6))))
    if nimg > 1:
        dt, res = run(nimg)
    g = gpu_out[:nimg].double().numpy()
    err = float(np.abs(g - res["out"]).max() / np.abs(res["out"]).max())
    # When the whole batch takes well under the target, repeat it so that the
    # figure rests on about target_s of CPU work.
    reps, total = 1, dt
    while total < target_s:
        more = max(1, int((target_s - total) / max(dt, 1e-6)))
        for _ in range(more):
            total += run(nimg)[0]
        reps += more
    tokens = reps * nimg * wl.height * wl.width
    return {
        "value": tokens / total,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{nimg} of {wl.batch} images of the same batch, run {reps} times "
                  f"({tokens} tokens), {total:.1f} s wall, fp64 C + OpenMP",
        "sample_max_rel_err_vs_gpu": err,
    }


def copy_calibration(dev, reps: int = COPY_REPS) -> None:
    """Run a plain device-to-device copy of COPY_BYTES a few times, so a
    counter run can scale the attention kernel's FETCH_SIZE / WRITE_SIZE by
    what the same counters read for a kernel of known traffic."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector
# the workloads whose lines are embedded under "configs" besides the headline
ALL_WORKLOADS = ("tiny_f32", "stage1", "stage2", "stage3", "highres")


def kernel_name(wl, shared_routing=False, kv_ratio=1) -> str:
    if image_path(wl, shared_routing, kv_ratio):
        return "image"
    return "small" if small_path(wl, shared_routing, kv_ratio) else "attend"


def roofline_entry(wl, attn_ms: float, ab: dict, shared_routing=False, kv_ratio=1) -> dict:
    """The bound of the forward's dominant kernel and how close it runs to it:
    HBM bytes for the memory-bound shapes, MFMA flops for the high-resolution
    attention (1024 keys per query: arithmetic intensity above the ridge)."""
    achieved_gbs = ab["attend"] / (attn_ms * 1e-3) / 1e9
    tflops = attention_flops(wl, kv_ratio) / (attn_ms * 1e-3) / 1e12
    mfma_bound = wl.dtype == "bf16" and wl.topk_effective * wl.tokens_per_region // \
        max(kv_ratio, 1) ** 2 >= 512
    if mfma_bound:
        return {"bound": "mfma", "kernel": kernel_name(wl, shared_routing, kv_ratio),
                "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / BF16_PEAK_TFLOPS, "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": ab["attend"]}
    peak_tf = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    return {"bound": "hbm", "kernel": kernel_name(wl, shared_routing, kv_ratio),
            "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS, "algorithmic_bytes": ab["attend"],
            "attention_tflops": tflops, "mfma_frac": tflops / peak_tf}


def measure(wl, args, want_graph: bool = True, keep_inputs: bool = False) -> dict:
    """Time args.steps forwards of workload wl (after args.warmup), rotating
    over enough buffer sets to miss the MALL; then the same forwards as a
    captured graph and once more with per-kernel events.  Inputs are already
    resident in HBM when the timed region starts."""
    import torch

    from vision_transformer_sparse_region_amd import bra
    from vision_transformer_sparse_region_amd.workloads import make_inputs, make_proj_weights

    dev = torch.device("cuda:0")
    host = make_inputs(wl)
    S = wl.tokens * wl.channels * (2 if wl.dtype == "bf16" else 4)
    nsets = args.buffer_sets or max(1, -(-2 * MALL_BYTES // (4 * S)))
    sets = []
    for i in range(nsets):
        d = {n: host[n].to(dev) for n in ("q", "k", "v", "lepe_w", "lepe_b")}
        d["out"] = torch.empty_like(d["q"])
        d["idx"] = torch.empty((wl.batch, 1 if args.shared_routing else wl.num_heads,
                                wl.regions, wl.topk_effective), dtype=torch.int32, device=dev)
        sets.append(d)

    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                wl.dtype, shared_routing=args.shared_routing,
                kv_downsample_ratio=args.kv_downsample, projections=args.projections)
    stream = torch.cuda.current_stream()
    wts = {n: t.to(dev) for n, t in make_proj_weights(wl).items()} if args.projections else None

    # Each set's C-ABI arguments are prepared once, as a C caller holds its
    # pointers: the timed loop makes the bra_forward call and nothing else on
    # the host (through the Python wrapper a call costs several microseconds
    # of tensor-to-pointer marshalling, more than the smallest workload's
    # kernel).
    lib = bra.load_library()
    if wts is not None:
        # the module input x is the q set; the handle stages q, k, v
        fwd = lib.bra_forward_proj
        argv = [(h.handle, d["q"].data_ptr(), wts["w_qkv"].data_ptr(), wts["b_qkv"].data_ptr(),
                 d["lepe_w"].data_ptr(), d["lepe_b"].data_ptr(), wts["w_o"].data_ptr(),
                 wts["b_o"].data_ptr(), d["out"].data_ptr(), d["idx"].data_ptr())
                for d in sets]
    else:
        fwd = lib.bra_forward
        argv = [(h.handle, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                 d["lepe_w"].data_ptr(), d["lepe_b"].data_ptr(), d["out"].data_ptr(),
                 d["idx"].data_ptr()) for d in sets]

    def step(i, s):
        st = fwd(*argv[i % nsets], s)
        if st != bra.BRA_OK:
            bra._check(st, fwd.__name__)

    s0 = stream.cuda_stream
    for i in range(args.warmup):
        step(i, s0)
    torch.cuda.synchronize()
    # Timed region: K back-to-back forwards between two events on the stream.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i, s0)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    # The same forwards captured once as a HIP graph (one forward per buffer
    # set) and replayed about K / sets times: the host's launch cost is gone.
    graph_ms = None
    if want_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            sc = torch.cuda.current_stream().cuda_stream  # the capture stream
            for i in range(nsets):
                step(i, sc)
        reps = max(1, args.steps // nsets)
        g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(end) / (reps * nsets)
        del g
    # Per-kernel breakdown: the same K forwards again, over the same buffer
    # sets, with the library recording HIP events on the launch stream before
    # the first kernel and after each of the three (event records between
    # kernels add a few microseconds per step, so this pass does not feed
    # `value`; it feeds the per-kernel times and the roofline).
    bra.bra_timing_enable(h.handle, args.steps)
    for i in range(args.steps):
        step(i, s0)
    times = bra.bra_timing_read(h.handle, args.steps)
    h.close()

    ms_per_step = gpu_ms / args.steps
    single = one_kernel(wl, args.shared_routing, args.kv_downsample) and not args.projections
    pool_ms = sum(t[0] for t in times) / len(times) if not single else None
    # (no routing kernel runs when the attention kernel routes: the interval
    # between its two events is empty)
    fused_route = route_in_attend(wl, args.shared_routing) or one_kernel(wl) or \
        (route_in_pool(wl, args.shared_routing) and not args.projections)
    route_ms = sum(t[1] for t in times) / len(times) if not fused_route else None
    attn_ms = sum(t[2] for t in times) / len(times)
    ab = algorithmic_bytes(wl, args.shared_routing, args.kv_downsample, args.projections)
    roof = roofline_entry(wl, attn_ms, ab, args.shared_routing, args.kv_downsample)
    total = ab["pool"] + ab["route"] + ab["attend"]
    roof["step_frac_hbm"] = total / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    if ab["pool"] and pool_ms:
        roof["pool_frac_hbm"] = ab["pool"] / (pool_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    res = {
        "workload": wl.name,
        "description": wl.description,
        "ms_per_step": ms_per_step,
        "value": wl.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "dtype": wl.dtype,
        "buffer_sets": nsets,
        "kernel_ms": {"region_pool": pool_ms, "route": route_ms,
                      (kernel_name(wl, args.shared_routing, args.kv_downsample)
                       if single else "attend"): attn_ms},
        "wall_s": wall,
        "roofline": roof,
    }
    if graph_ms is not None:
        res["graph"] = {"ms_per_step": graph_ms, "value": wl.tokens / (graph_ms * 1e-3),
                        "unit": "tokens/s", "forwards_per_graph": nsets}
    if keep_inputs:
        res["_host"] = host
        res["_last_out"] = sets[(args.steps - 1) % nsets]["out"].cpu()
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="stage1")
    ap.add_argument("--buffer-sets", type=int, default=0,
                    help="input/output sets to rotate over (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the pass that replays the forwards as one captured HIP graph")
    ap.add_argument("--no-all-configs", action="store_true",
                    help="time only the headline workload (by default the other workloads "
                         "of the benchmark table are timed too and embedded under 'configs')")
    ap.add_argument("--shared-routing", action="store_true",
                    help="one routing per region for every head (full-C region affinity)")
    ap.add_argument("--kv-downsample", type=int, default=1,
                    help="KV downsampling ratio r (attention over r x r average-pooled K/V)")
    ap.add_argument("--projections", action="store_true",
                    help="time bra_forward_proj: the module's qkv and output projections "
                         "around the path (random bf16 weights)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run a {COPY_BYTES >> 20} MiB device copy (for counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this implementation runs on one GPU; the forward needs no collective and "
              "its multi-GPU sharding is described but not built.", file=sys.stderr)
        return 2

    import torch

    from vision_transformer_sparse_region_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    res = measure(wl, args, want_graph=not args.no_graph, keep_inputs=True)
    if args.copy_calibration:
        copy_calibration(dev)
    roof = dict(res["roofline"])
    # (counter summaries exist for the plain forward of each workload)
    plain = not (args.projections or args.shared_routing or args.kv_downsample > 1)
    roof["traffic"] = stored_traffic(wl.name, roof["kernel"]) if plain else None
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.description,
            "batch": wl.batch, "height": wl.height, "width": wl.width,
            "channels": wl.channels, "num_heads": wl.num_heads, "n_win": wl.n_win,
            "topk": wl.topk, "buffer_sets": res["buffer_sets"],
            "routing": "shared by all heads" if args.shared_routing else "per head",
            "kv_downsample_ratio": args.kv_downsample,
            "projections": bool(args.projections),
            **({"output_projection": "attention epilogue" if out_proj_in_attend(wl)
                else "own kernel"} if args.projections else {}),
            "kernel_ms": res["kernel_ms"],
            "wall_s": res["wall_s"],
        },
        "roofline": roof,
    }
    if "graph" in res:
        line["graph"] = res["graph"]
    # the other workloads of the benchmark table, the same variant, timed over
    # at least CONFIG_MIN_STEPS steps after at least CONFIG_MIN_WARMUP untimed
    # ones: a few warm-up forwards of the shorter workloads leave the core
    # clock below its loaded rate (the high-res attention ran ~10% slower)
    if not args.no_all_configs:
        configs = {}
        cargs = argparse.Namespace(**vars(args))
        cargs.steps = max(args.steps, CONFIG_MIN_STEPS)
        cargs.warmup = max(args.warmup, CONFIG_MIN_WARMUP)
        for name in ALL_WORKLOADS:
            if name == args.workload:
                continue
            r = measure(WORKLOADS[name], cargs, want_graph=False)
            configs[name] = {k: r[k] for k in ("description", "ms_per_step", "value", "unit",
                                              "dtype", "kernel_ms", "roofline")}
            configs[name]["steps"] = cargs.steps
            configs[name]["warmup"] = cargs.warmup
            configs[name]["roofline"] = dict(r["roofline"])
            configs[name]["roofline"]["traffic"] = \
                stored_traffic(name, r["roofline"]["kernel"]) if plain else None
        line["configs"] = configs
    if not args.no_cpu_baseline and not args.projections:
        line["cpu_baseline"] = cpu_baseline(wl, res["_host"], res["_last_out"],
                                            shared=args.shared_routing,
                                            kv_ratio=args.kv_downsample)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
