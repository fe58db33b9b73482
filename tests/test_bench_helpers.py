"""Host-side pieces of bench.py: the byte counts the roofline divides by, the
committed traffic summary it reads, and the refusal of more than one GPU."""
import os

import bench
from vision_transformer_sparse_region_amd.workloads import WORKLOADS


def test_algorithmic_bytes_stage1():
    wl = WORKLOADS["stage1"]
    ab = bench.algorithmic_bytes(wl)
    S = 64 * 56 * 56 * 64 * 2
    M = 64 * 2 * 49 * 32 * 8
    idx = 64 * 2 * 49 * 1 * 4
    assert ab["S"] == S
    # 49 regions, 2 heads: routed inside the attention kernel, which also sums
    # the Q means; the pool kernel reads k and writes the K means only, in
    # fp64 and (64-token windows) in fp32, and the attention kernel reads the
    # fp32 ones
    assert bench.kmean32(wl)
    assert ab["pool"] == S + M + M // 2
    assert ab["route"] == 0
    assert ab["attend"] == 4 * S + M // 2 + idx + 64 * 26 * 4


def test_fp32_k_means_only_for_windows_of_32_tokens():
    assert not bench.kmean32(WORKLOADS["stage2"])            # 16-token windows
    assert not bench.kmean32(WORKLOADS["stage3"])            # routed outside
    assert not bench.kmean32(WORKLOADS["highres"])           # 256 regions
    assert not bench.kmean32(WORKLOADS["stage1"], shared_routing=True)
    wl = WORKLOADS["stage2"]
    S = 64 * 28 * 28 * 128 * 2
    M = 64 * 128 * 49 * 8
    ab = bench.algorithmic_bytes(wl)
    assert ab["pool"] == S + M


def test_q_means_summed_in_attention_kernel():
    # every query tile of a region is some wave's first job (at most 4 jobs)
    assert bench.qmean_in_attend(WORKLOADS["stage1"])       # 2 heads x 2 groups of 2 tiles
    assert bench.qmean_in_attend(WORKLOADS["stage2"])       # 4 heads x 1 tile
    assert not bench.qmean_in_attend(WORKLOADS["stage3"])   # 8 heads: routed separately
    assert not bench.qmean_in_attend(WORKLOADS["tiny_f32"])  # fp32
    assert not bench.qmean_in_attend(WORKLOADS["stage1"], shared_routing=True)
    base = WORKLOADS["stage1"]
    assert bench.qmean_in_attend(base.with_(height=56, width=42))       # t = 48: 2 + 1 tiles
    assert not bench.qmean_in_attend(base.with_(height=42, width=42,    # t = 36, 3 heads:
                                                 channels=96, num_heads=3, n_win=7))  # 6 jobs
    assert not bench.qmean_in_attend(base.with_(height=70, width=70))   # t = 100: 8 jobs


def test_algorithmic_bytes_highres_separate_route():
    wl = WORKLOADS["highres"]
    ab = bench.algorithmic_bytes(wl)
    S = 8 * 128 * 128 * 64 * 2
    M = 8 * 2 * 256 * 32 * 8
    idx = 8 * 2 * 256 * 16 * 4
    assert ab["route"] == 2 * M + idx
    assert ab["attend"] == 4 * S + idx + 64 * 26 * 4


def test_algorithmic_bytes_stage3_means_and_routing_in_one_kernel():
    wl = WORKLOADS["stage3"]
    assert bench.route_in_pool(wl)
    ab = bench.algorithmic_bytes(wl)
    S = 64 * 14 * 14 * 256 * 2
    idx = 64 * 8 * 49 * 16 * 4
    # one kernel reads q and k and writes the ids; the means stay on chip
    assert ab["pool"] == 2 * S + idx
    assert ab["route"] == 0
    assert ab["attend"] == 4 * S + idx + 256 * 26 * 4
    # the other shapes keep their kernels
    assert not bench.route_in_pool(WORKLOADS["stage1"])    # routed in the attention kernel
    assert not bench.route_in_pool(WORKLOADS["highres"])   # 256 regions
    assert not bench.route_in_pool(WORKLOADS["tiny_f32"])  # fp32
    assert not bench.route_in_pool(wl, shared_routing=True)


def test_attention_flops_highres():
    wl = WORKLOADS["highres"]
    # 4 * tokens * heads * k * t * head_dim
    assert bench.attention_flops(wl) == 4.0 * 8 * 128 * 128 * 2 * 16 * 64 * 32


def test_traffic_summary_parses_and_matches_sources():
    path = bench.traffic_summary_path("stage1")
    if not os.path.exists(path):
        return
    rec = bench.read_traffic_record(path)
    assert rec["workload"] == "stage1" and rec["kernel"] == "attend"
    assert rec["hbm_bytes_per_launch"] > 0
    # the stored figure is used only while the kernel sources are unchanged
    expect = rec["hbm_bytes_per_launch"] if rec["kernel_source_sha256_16"] == \
        bench.kernel_source_hash() else None
    assert bench.stored_traffic("stage1") == expect


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // one\n    return x + 1; /* two */\n}\n"
    b = "// header\nint f(int x) {\n\n    return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
