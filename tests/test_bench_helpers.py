"""Host-side pieces of bench.py: the byte counts the roofline divides by, the
committed traffic summary it reads, and the refusal of more than one GPU."""
import glob
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
    # stage 2 without the whole-image kernel (head-shared routing): the pool
    # kernel reads k and writes the K means, fp64 only
    wl = WORKLOADS["stage2"]
    S = 64 * 28 * 28 * 128 * 2
    M = 64 * 128 * 49 * 8
    ab = bench.algorithmic_bytes(wl, kv_ratio=2)
    assert ab["pool"] == S + M + 2 * S + 2 * S // 4


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


def test_algorithmic_bytes_whole_image_kernel():
    """Stages 2 and 3 run one kernel per (image, head group): q, k and v are
    read once and out written once; the means and the routing stay on chip
    and only the ids are exported."""
    for name, C, H, heads, k in (("stage2", 128, 28, 4, 4), ("stage3", 256, 14, 8, 16)):
        wl = WORKLOADS[name]
        assert bench.image_path(wl)
        ab = bench.algorithmic_bytes(wl)
        S = 64 * H * H * C * 2
        idx = 64 * heads * 49 * k * 4
        assert ab["pool"] == 0 and ab["route"] == 0
        assert ab["attend"] == 4 * S + idx + C * 26 * 4
        assert bench.kernel_name(wl) == "image"
    # the other shapes and variants keep their kernels
    assert not bench.image_path(WORKLOADS["stage1"])
    assert not bench.image_path(WORKLOADS["highres"])
    assert not bench.image_path(WORKLOADS["tiny_f32"])
    assert not bench.image_path(WORKLOADS["stage3"], shared_routing=True)
    assert not bench.image_path(WORKLOADS["stage2"], kv_ratio=2)
    assert not bench.image_path(WORKLOADS["stage2"].with_(topk=6))
    # stage 3 with head-shared routing: means and routing in the pool kernel
    assert bench.route_in_pool(WORKLOADS["stage3"]) and \
        not bench.route_in_pool(WORKLOADS["stage3"], shared_routing=True)


def test_algorithmic_bytes_small_fp32_kernel():
    """The tiny fp32 problem (49 regions x 2 heads = 98 workgroups) runs the
    one-launch kernel: q, k, v read once, out written once, the ids exported.
    Larger fp32 problems, KV downsampling and shared routing keep the
    pool/routing/attention kernels."""
    wl = WORKLOADS["tiny_f32"]
    assert bench.small_path(wl) and bench.kernel_name(wl) == "small"
    ab = bench.algorithmic_bytes(wl)
    S = 28 * 28 * 64 * 4
    assert ab["pool"] == 0 and ab["route"] == 0
    assert ab["attend"] == 4 * S + 2 * 49 * 4 * 4 + 64 * 26 * 4
    assert bench.small_lds_bytes(wl) <= 160 * 1024
    assert not bench.small_path(WORKLOADS["stage1"])
    assert not bench.small_path(wl.with_(batch=4, channels=128, num_heads=4))  # 784 triples
    assert not bench.small_path(wl, kv_ratio=2)
    assert not bench.small_path(wl, shared_routing=True)


def test_roofline_bound_per_workload():
    """HBM for the memory-bound shapes, the bf16 MFMA peak for the
    high-resolution attention (1024 keys per query)."""
    for name in ("stage1", "stage2", "stage3", "tiny_f32"):
        wl = WORKLOADS[name]
        r = bench.roofline_entry(wl, 0.03, bench.algorithmic_bytes(wl))
        assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    wl = WORKLOADS["highres"]
    r = bench.roofline_entry(wl, 0.08, bench.algorithmic_bytes(wl))
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - bench.attention_flops(wl) / 0.08e-3 / 1e12 / 2500.0) < 1e-12


def test_attention_flops_highres():
    wl = WORKLOADS["highres"]
    # 4 * tokens * heads * k * t * head_dim
    assert bench.attention_flops(wl) == 4.0 * 8 * 128 * 128 * 2 * 16 * 64 * 32


def test_traffic_summaries_parse_and_match_sources():
    """Every committed traffic summary names its workload and kernel, and its
    figure is used only while that kernel's sources are unchanged."""
    for path in glob.glob(os.path.join(bench.PROFILES, "*_traffic.md")):
        rec = bench.read_traffic_record(path)
        kernel, wl = rec["kernel"], rec["workload"]
        assert os.path.basename(path) == f"{kernel}_{wl}_traffic.md"
        assert rec["hbm_bytes_per_launch"] > 0
        expect = rec["hbm_bytes_per_launch"] if rec["kernel_source_sha256_16"] == \
            bench.kernel_source_hash(kernel) else None
        assert bench.stored_traffic(wl, kernel) == expect


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // one\n    return x + 1; /* two */\n}\n"
    b = "// header\nint f(int x) {\n\n    return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
