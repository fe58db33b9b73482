"""GPU: the path with the module's qkv and output projections on either side
(bra_forward_proj) against the CPU oracle, through the C ABI.

The qkv projection rounds q, k, v once to bf16, as the module's Linear layer
would.  The GPU sums each output in fp32 on the MFMA before that rounding;
the oracle sums in fp64.  So a value lying within about 2^-16 of a bf16
rounding boundary can round one step apart on the two sides (about one
element in a thousand).  Such a step moves a region mean by about 6e-5 and an
affinity by well under 1e-4 of the row's largest.  Routing is therefore
compared with that looser near-tie bound: an index that differs must have an
affinity within 1e-3 of the row's largest |A| of the oracle's choice.  The
output is compared with the oracle's projections evaluated on the GPU's
routing, against the bf16 bound.  With identity weights the projected path
must equal bra_forward of (x, x, x) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, max_rel_err, oracle_cfg, say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import (WORKLOADS, Workload, make_inputs,
                                                           make_proj_weights)

pytestmark = pytest.mark.gpu

PROJ_TIE = 1e-3


def _handle(wl, projections=True, shared=False, kv=1):
    return bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                   wl.dtype, shared_routing=shared, kv_downsample_ratio=kv,
                   projections=projections)


def _run_proj(wl, x, wts, lepe_w, lepe_b):
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in wts.items()}
    with _handle(wl) as h:
        out, idx = h.forward_proj(x.to(dev), g["w_qkv"], g["w_o"], g["b_qkv"], g["b_o"],
                                  lepe_w.to(dev), lepe_b.to(dev))
        torch.cuda.synchronize()
    return out.cpu(), idx.cpu().numpy()


CASES = [
    Workload("proj_stage1_b4", 4, 56, 56, 64, 2, 7, 1, "bf16", 401),
    Workload("proj_stage2_b2", 2, 28, 28, 128, 4, 7, 4, "bf16", 402, lepe_bias=True),
    Workload("proj_stage3_b2", 2, 14, 14, 256, 8, 7, 16, "bf16", 403),
    Workload("proj_ragged_t15", 2, 12, 20, 64, 2, 4, 3, "bf16", 404, lepe_bias=True),
    Workload("proj_r100", 1, 40, 40, 96, 3, 10, 5, "bf16", 405),
    # the output projection as its own kernel (C > 8 t): ragged last row slice,
    # one head (half a channel chunk), C > 256 (32-token slices), stage 4
    Workload("proj_out_ragged_rows", 1, 10, 10, 128, 4, 5, 3, "bf16", 408, lepe_bias=True),
    Workload("proj_one_head_t2", 3, 8, 4, 32, 1, 4, 2, "bf16", 409),
    Workload("proj_wide_c320", 1, 14, 14, 320, 10, 7, 4, "bf16", 410),
    Workload("proj_stage4_b2", 2, 7, 7, 512, 16, 7, 49, "bf16", 411),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_projected_forward_matches_oracle(wl):
    inp = make_inputs(wl)
    wts = make_proj_weights(wl)
    say(f"[gpu] proj {wl.name}: B={wl.batch} {wl.height}x{wl.width} C={wl.channels} "
        f"heads={wl.num_heads} n_win={wl.n_win} topk={wl.topk}")
    gout, gidx = _run_proj(wl, inp["q"], wts, inp["lepe_w"], inp["lepe_b"])
    cfg = oracle_cfg(wl, 0.0)
    f = {n: t.double().numpy() for n, t in wts.items()}
    x = inp["q"].double().numpy()
    lw, lb = inp["lepe_w"].double().numpy(), inp["lepe_b"].double().numpy()
    res = oracle.bra_forward_proj(cfg, 1, x, f["w_qkv"], f["b_qkv"], lw, lb, f["w_o"], f["b_o"],
                                  want_qkv=True)
    # routing: equal up to affinities within PROJ_TIE of the row's largest |A|
    C = wl.channels
    qkv = res["qkv"]
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    means = oracle.bra_forward(cfg, q, k, v, want_aff=True)
    aff, oidx = means["aff"], res["idx"]
    assert (means["idx"] == oidx).all()
    ties = 0
    for b, h, r, j in np.argwhere(gidx != oidx):
        row = aff[b, h, r]
        gap = abs(row[gidx[b, h, r, j]] - row[oidx[b, h, r, j]])
        assert gap <= PROJ_TIE * np.abs(row).max(), (wl.name, b, h, r, j, gap)
        ties += 1
    # output: the oracle's projections, attention on the GPU's routing, the
    # output projection
    y = oracle.attend_with_routing(cfg, q, k, v, lw, lb, gidx)
    ref = oracle.linear(y, f["w_o"], f["b_o"])
    err = max_rel_err(gout, ref)
    say(f"[gpu] proj {wl.name}: max rel err {err:.3e} (bound {TOL['bf16']:g}), "
        f"routing differences within the projection bound: {ties}")
    assert err <= TOL["bf16"], (wl.name, err)


@pytest.mark.parametrize("wl", [WORKLOADS["stage1"].with_(batch=4),
                                Workload("eye_generic", 2, 12, 20, 64, 2, 4, 3, "bf16", 406),
                                WORKLOADS["stage3"].with_(batch=2),
                                Workload("eye_generic_small_t", 1, 10, 10, 128, 4, 5, 3, "bf16",
                                         412)],
                         ids=["stage1_b4", "generic", "stage3_b2", "generic_small_t"])
def test_identity_projections_equal_plain_forward(wl):
    """w_qkv = [I; I; I], w_o = I, no biases: q = k = v = x exactly, and
    out = bf16(y), the plain forward's own rounding -- bit for bit, with the
    output projection in the attention epilogue (stage 1, generic) and as
    its own kernel (stage 3, generic with small regions)."""
    inp = make_inputs(wl)
    C = wl.channels
    eye = torch.eye(C, dtype=torch.bfloat16)
    dev = torch.device("cuda:0")
    x = inp["q"].to(dev)
    lw, lb = inp["lepe_w"].to(dev), inp["lepe_b"].to(dev)
    say(f"[gpu] identity projections: {wl.name}")
    with _handle(wl) as h:
        a, ia = h.forward_proj(x, torch.cat([eye, eye, eye]).to(dev), eye.to(dev), None, None,
                               lw, lb)
    with _handle(wl, projections=False) as h:
        b, ib = h.forward(x, x, x, lw, lb)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ia, ib)


def test_projection_argument_checks():
    wl = Workload("checks", 1, 28, 28, 64, 2, 7, 1, "bf16", 407)
    dev = torch.device("cuda:0")
    x = torch.zeros((1, 28, 28, 64), dtype=torch.bfloat16, device=dev)
    w3 = torch.zeros((192, 64), dtype=torch.bfloat16, device=dev)
    wo = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(x)
    with _handle(wl, projections=False) as h:
        assert bra.bra_forward_proj_status(h.handle, x, w3, None, None, None, wo, None, out) == \
            bra.BRA_ERR_UNSUPPORTED
    with _handle(wl) as h:
        assert bra.bra_forward_proj_status(h.handle, x, None, None, None, None, wo, None,
                                           out) == bra.BRA_ERR_NULL
        assert bra.bra_forward_proj_status(h.handle, x, w3, None, None, None, wo, None, x) == \
            bra.BRA_ERR_ALIAS
        assert bra.bra_forward_proj_status(h.handle, x, w3, None, None, None, wo, None,
                                           out) == bra.BRA_OK
        torch.cuda.synchronize()
