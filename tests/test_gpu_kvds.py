"""GPU parity of KV downsampling (bra_config_t.kv_downsample_ratio r > 1: the
attention gathers K and V average-pooled over r x r blocks, routing and LePE
stay at full resolution [P1 §4.1]) through the C ABI, against the oracle's
oracle_bra_forward_kvds.  Same bar as tests/parity.py: routing bit-exact up to
logged near-ties, outputs within the dtype's bound (the pooled K/V are
rounded once to the I/O type, as the inputs are)."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, check_routing, max_rel_err, oracle_cfg, say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    (WORKLOADS["highres"].with_(batch=1, seed=401), 4),
    (WORKLOADS["highres"].with_(batch=1, seed=402), 2),
    (WORKLOADS["stage1"].with_(batch=4, seed=403), 2),
    (WORKLOADS["stage1"].with_(batch=4, seed=404), 8),
    (WORKLOADS["stage2"].with_(batch=4, seed=405), 4),
    (Workload("kvds_ragged_bias", 2, 24, 16, 64, 2, 4, 3, "bf16", 406, lepe_bias=True), 2),
    (Workload("kvds_f32", 2, 28, 28, 64, 2, 7, 4, "f32", 407, lepe_bias=True), 2),
    (Workload("kvds_f32_r4", 2, 28, 28, 64, 2, 7, 4, "f32", 408), 4),
    # "从静态到动态" §4.1: dim 128, n_win 7, topk 4, kv_downsample_ratio 4 (4 heads
    # of 32, a 56 x 56 map): tiles above 64 KB of LDS
    (Workload("page_dim128", 2, 56, 56, 128, 4, 7, 4, "bf16", 409, lepe_bias=True), 4),
]


def run_gpu_kvds(wl: Workload, inp: dict, ratio: int):
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w, b = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                wl.dtype, kv_downsample_ratio=ratio)
    try:
        out, idx = h.forward(q, k, v, w, b)
        out2 = h.forward_routed(q, k, v, idx, w, b)
        torch.cuda.synchronize()
    finally:
        h.close()
    return out.cpu(), idx.cpu().numpy(), out2.cpu()


@pytest.mark.parametrize("wl,ratio", CASES, ids=[f"{w.name}_r{r}" for w, r in CASES])
def test_kv_downsampling_matches_oracle(wl, ratio):
    inp = make_inputs(wl)
    say(f"[gpu] kvds {wl.name} r={ratio}: B={wl.batch} {wl.height}x{wl.width} "
        f"C={wl.channels} heads={wl.num_heads} n_win={wl.n_win} topk={wl.topk} {wl.dtype}")
    out, gidx, out2 = run_gpu_kvds(wl, inp, ratio)
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v", "lepe_w", "lepe_b")}
    cfg = oracle_cfg(wl)
    res = oracle.bra_forward_kvds(cfg, ratio, f["q"], f["k"], f["v"], f["lepe_w"], f["lepe_b"])
    # routing is the full-resolution one: check it with the affinities of the plain forward
    aff = oracle.bra_forward(cfg, f["q"], f["k"], f["v"], want_aff=True)["aff"]
    ties = check_routing(gidx, {"idx": res["idx"], "aff": aff})
    assert not ties, "near-ties would need the downsampled attention on the GPU's routing"
    err = max_rel_err(out, res["out"], wl.num_heads)
    say(f"[gpu] kvds {wl.name} r={ratio}: max rel err {err:.3e} (bound {TOL[wl.dtype]:g})")
    assert err <= TOL[wl.dtype]
    # the routed entry point on the forward's own routing gives the same output
    assert torch.equal(out.view(torch.int16) if wl.dtype == "bf16" else out,
                       out2.view(torch.int16) if wl.dtype == "bf16" else out2)


def test_kv_downsampling_with_shared_routing():
    """Head-shared routing and KV downsampling together: the shared routing,
    then every head over the downsampled K/V of the shared routed regions."""
    wl = WORKLOADS["stage2"].with_(batch=2, seed=409)
    ratio = 2
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w, b = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    say("[gpu] kvds + shared routing")
    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                shared_routing=True, kv_downsample_ratio=ratio)
    try:
        out, idx = h.forward(q, k, v, w, b)
        torch.cuda.synchronize()
    finally:
        h.close()
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v", "lepe_w", "lepe_b")}
    cfg = oracle_cfg(wl)
    res = oracle.bra_forward_shared(cfg, f["q"], f["k"], f["v"], want_aff=True)
    gidx = idx.cpu().numpy()
    ties = check_routing(gidx, {"idx": res["idx"][:, None], "aff": res["aff"][:, None]})
    full = np.ascontiguousarray(np.repeat(gidx, wl.num_heads, axis=1))
    ref = oracle.attend_kvds(cfg, ratio, f["q"], f["k"], f["v"], full) + \
        oracle.lepe(cfg, f["v"], f["lepe_w"], f["lepe_b"])
    err = max_rel_err(out.cpu(), ref, wl.num_heads)
    say(f"[gpu] kvds + shared routing: max rel err {err:.3e}, near-ties {len(ties)}")
    assert err <= TOL[wl.dtype]


def test_routed_entry_with_kv_downsampling():
    """bra_forward_routed on random routings with KV downsampling."""
    wl = WORKLOADS["highres"].with_(batch=1, seed=410)
    ratio = 4
    inp = make_inputs(wl)
    rng = np.random.default_rng(410)
    idx = rng.integers(0, wl.regions, size=(1, 2, wl.regions, wl.topk_effective)).astype(np.int32)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w, b = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    say("[gpu] kvds routed entry")
    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                kv_downsample_ratio=ratio)
    try:
        out = h.forward_routed(q, k, v, torch.from_numpy(idx).to(dev), w, b)
        torch.cuda.synchronize()
    finally:
        h.close()
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v", "lepe_w", "lepe_b")}
    cfg = oracle_cfg(wl)
    ref = oracle.attend_kvds(cfg, ratio, f["q"], f["k"], f["v"], idx) + \
        oracle.lepe(cfg, f["v"], f["lepe_w"], f["lepe_b"])
    err = max_rel_err(out.cpu(), ref, wl.num_heads)
    say(f"[gpu] kvds routed entry: max rel err {err:.3e}")
    assert err <= TOL[wl.dtype]
