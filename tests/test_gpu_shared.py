"""GPU parity of head-shared routing (bra_config_t.shared_routing = 1; one
routing per region from the region means over all C channels, used by every
head [P1 §2.2; P2 §2.1; P3 §2.1; P4 §1.2]) through the C ABI, against the
oracle's oracle_bra_forward_shared.  Same bar as tests/parity.py: routing
bit-exact up to logged near-ties, outputs within the dtype's bound."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, check_routing, max_rel_err, oracle_cfg, say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    WORKLOADS["stage1"].with_(batch=4, seed=301),
    WORKLOADS["stage2"].with_(batch=4, seed=302),
    WORKLOADS["stage3"].with_(batch=4, seed=303),
    WORKLOADS["highres"].with_(batch=1, seed=304),
    Workload("shared_ragged_bias", 2, 12, 20, 64, 2, 4, 3, "bf16", 305, lepe_bias=True),
    Workload("shared_sixteen_heads", 2, 7, 7, 512, 16, 7, 49, "bf16", 306),
    Workload("shared_three_heads_t36", 2, 24, 24, 96, 3, 4, 5, "bf16", 307),
    Workload("shared_f32", 2, 28, 28, 64, 2, 7, 4, "f32", 308, lepe_bias=True),
    Workload("shared_r100", 2, 40, 40, 128, 4, 10, 3, "bf16", 310),
]


def check_shared(wl: Workload, inp: dict | None = None):
    inp = inp if inp is not None else make_inputs(wl)
    say(f"[gpu] shared {wl.name}: B={wl.batch} {wl.height}x{wl.width} C={wl.channels} "
        f"heads={wl.num_heads} n_win={wl.n_win} topk={wl.topk} {wl.dtype} seed={wl.seed}")
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w, b = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                wl.dtype, shared_routing=True)
    try:
        out, idx = h.forward(q, k, v, w, b)
        torch.cuda.synchronize()
    finally:
        h.close()
    out, gidx = out.cpu(), idx.cpu().numpy()
    assert gidx.shape[1] == 1
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v", "lepe_w", "lepe_b")}
    cfg = oracle_cfg(wl)
    res = oracle.bra_forward_shared(cfg, f["q"], f["k"], f["v"], f["lepe_w"], f["lepe_b"],
                                    want_aff=True)
    ties = check_routing(gidx, {"idx": res["idx"][:, None], "aff": res["aff"][:, None]})
    ref = res["out"]
    if ties:
        full = np.ascontiguousarray(np.repeat(gidx, wl.num_heads, axis=1))
        ref = oracle.attend_with_routing(cfg, f["q"], f["k"], f["v"], f["lepe_w"], f["lepe_b"],
                                         full)
    err = max_rel_err(out, ref, wl.num_heads)
    say(f"[gpu] shared {wl.name}: max rel err {err:.3e} (bound {TOL[wl.dtype]:g}), "
        f"near-ties {len(ties)}")
    assert err <= TOL[wl.dtype]
    return gidx


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_shared_routing_matches_oracle(wl):
    check_shared(wl)


def test_shared_exact_ties_pick_lower_regions():
    wl = Workload("shared_all_tied", 2, 28, 28, 128, 4, 7, 6, "bf16", 309)
    inp = make_inputs(wl)
    tile = inp["k"][:, :4, :4, :].clone()
    inp["k"] = tile.repeat(1, 7, 7, 1).contiguous()
    idx = check_shared(wl, inp)
    assert (idx == np.arange(6, dtype=np.int32)).all()


def test_shared_routing_reused_by_forward_routed():
    """A shared routing ([B, 1, R, k]) given back to bra_forward_routed
    reproduces the forward's output."""
    wl = WORKLOADS["stage2"].with_(batch=2, seed=310)
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w, b = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    say("[gpu] shared routing through forward_routed")
    h = bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                shared_routing=True)
    try:
        out, idx = h.forward(q, k, v, w, b)
        out2 = h.forward_routed(q, k, v, idx, w, b)
        torch.cuda.synchronize()
    finally:
        h.close()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
