"""GPU: the path with the module's qkv and output projections on either side
(bra_forward_proj) against the CPU oracle, through the C ABI.

The qkv projection rounds q, k, v once to bf16, as the module's Linear layer
would.  The GPU sums each output in fp32 on the MFMA before that rounding;
the oracle sums in fp64.  So a value lying within about 2^-16 of a bf16
rounding boundary can round one step apart on the two sides (about one
element in a thousand).  The test therefore checks each stage on its own:
  * the GPU's projected q, k, v (bra_debug_projected_qkv) against the
    oracle's fp64 sums element by element, within the fp32 summation bound
    gamma_K (sum |x w| + |b|) plus half a bf16 step; elements whose rounding
    differs from the oracle's (flips: mostly one step, more where the sum
    cancels) are counted and must stay rare;
  * the routing against the oracle run on the GPU's own q, k, v, with the
    standard bar (bit-exact up to logged near-ties within 1e-6 of the row's
    largest |A|);
  * the output against the oracle's attention and output projection on the
    GPU's q, k, v and routing, and end to end against the oracle's own
    projections on the GPU's routing, both within the bf16 bound.
With identity weights the projected path must equal bra_forward of (x, x, x)
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, check_routing, max_rel_err, oracle_cfg, say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import (WORKLOADS, Workload, make_inputs,
                                                           make_proj_weights)

pytestmark = pytest.mark.gpu

FLIP_FRACTION = 5e-3  # at most this share of q/k/v elements rounded apart


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
        q, k, v = h.projected_qkv()
        torch.cuda.synchronize()
    return out.cpu(), idx.cpu().numpy(), [t.cpu() for t in (q, k, v)]


def _check_projection(name, gpu, rounded, exact, bound):
    """One projected map against the oracle: `rounded` is the oracle's bf16
    value, `exact` its fp64 sum before rounding, `bound` the fp32 summation
    error bound of each element (gamma_K (sum |x w| + |b|)).  The GPU's fp32
    sum lies within `bound` of `exact`, and rounding it adds at most half a
    bf16 step: every element must lie within that, and elements that differ
    from the oracle's rounding (flips) are counted."""
    g = gpu.double().numpy()
    mag = np.abs(exact) + bound
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7)
    excess = np.abs(g - exact) - (bound + 0.5 * ulp)
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, (f"{name}: {g[worst]!r} vs exact {exact[worst]!r} "
                                f"(bound {bound[worst]:.3g}) at {worst}")
    return int((g != rounded).sum())


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
    gout, gidx, gqkv = _run_proj(wl, inp["q"], wts, inp["lepe_w"], inp["lepe_b"])
    cfg = oracle_cfg(wl, 0.0)
    f = {n: t.double().numpy() for n, t in wts.items()}
    x = inp["q"].double().numpy()
    lw, lb = inp["lepe_w"].double().numpy(), inp["lepe_b"].double().numpy()
    res = oracle.bra_forward_proj(cfg, 1, x, f["w_qkv"], f["b_qkv"], lw, lb, f["w_o"], f["b_o"],
                                  want_qkv=True)
    C = wl.channels
    qkv = res["qkv"]
    oq, ok, ov = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    # 1. the projections, element by element, against the fp64 sums and the
    #    fp32 summation bound (K = C products and a bias, unit roundoff 2^-24)
    exact = oracle.linear(x, f["w_qkv"], f["b_qkv"])
    u = 2.0 ** -24
    gamma = (C + 1) * u / (1 - (C + 1) * u)
    mags = np.abs(x).reshape(-1, C) @ np.abs(f["w_qkv"]).T + np.abs(f["b_qkv"])
    bound = gamma * mags.reshape(exact.shape)
    flips = 0
    for i, (name, gt, ot) in enumerate((("q", gqkv[0], oq), ("k", gqkv[1], ok),
                                        ("v", gqkv[2], ov))):
        sl = slice(i * C, (i + 1) * C)
        flips += _check_projection(f"{wl.name}: {name}", gt, ot, exact[..., sl], bound[..., sl])
    share = flips / (3 * oq.size)
    assert share <= FLIP_FRACTION, f"{wl.name}: {flips} one-step flips ({share:.2e} of q/k/v)"
    # 2. the routing on the GPU's own q, k, v: the standard bar
    gq, gk, gv = (t.double().numpy() for t in gqkv)
    own = oracle.bra_forward(cfg, gq, gk, gv, want_aff=True)
    ties = check_routing(gidx, own)
    # 3. the output: on the GPU's q, k, v and routing, then end to end
    y = oracle.attend_with_routing(cfg, gq, gk, gv, lw, lb, gidx)
    err = max_rel_err(gout, oracle.linear(y, f["w_o"], f["b_o"]), wl.num_heads)
    y_e2e = oracle.attend_with_routing(cfg, oq, ok, ov, lw, lb, gidx)
    err_e2e = max_rel_err(gout, oracle.linear(y_e2e, f["w_o"], f["b_o"]), wl.num_heads)
    say(f"[gpu] proj {wl.name}: q/k/v one-step flips {flips} ({share:.1e}), near-ties "
        f"{len(ties)}, max rel err {err:.3e} on the GPU's q/k/v, {err_e2e:.3e} end to end "
        f"(bound {TOL['bf16']:g})")
    assert err <= TOL["bf16"], (wl.name, err)
    assert err_e2e <= TOL["bf16"], (wl.name, err_e2e)


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
        assert bra.bra_debug_projected_qkv_status(h.handle, x, x, x) == bra.BRA_ERR_UNSUPPORTED
    with _handle(wl) as h:
        assert bra.bra_forward_proj_status(h.handle, x, None, None, None, None, wo, None,
                                           out) == bra.BRA_ERR_NULL
        assert bra.bra_forward_proj_status(h.handle, x, w3, None, None, None, wo, None, x) == \
            bra.BRA_ERR_ALIAS
        assert bra.bra_forward_proj_status(h.handle, x, w3, None, None, None, wo, None,
                                           out) == bra.BRA_OK
        torch.cuda.synchronize()
