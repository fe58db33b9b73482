"""GPU: the routing's fp32 shortcuts and their exact fallbacks.  The top-k
sorts fp32 keys first and falls back to the exact fp64 sort when the fp32
keys of the leading positions are not strictly decreasing; the routing inside
the attention kernel also screens with fp32 K means and an error bound, and
reads the fp64 means when the bound cannot separate the leaders.  Two regions whose K means differ by 2^-31 in one dim per head
have affinities that differ by about 1e-10 of their size: distinct in fp64,
one fp32 key.  Made the two best regions of every row (large, equal K
everywhere else; Q biased positive), their order must still be the oracle's
fp64 order, exactly -- the near-tie tolerance of the other parity tests
would accept either order, so this test compares the ids bit for bit.
Covered: routing inside the attention kernel (k = 4 on 16-token windows,
exact pass only; k = 1 and k = 4 on 64- and 36-token windows, screened), the
means-and-routing kernel (k = 16), and the routing kernel over 100 regions
(two entries per lane).  A last case makes the fp32 products
overflow (K and Q means near 2^70): finite in fp64, infinite in fp32, so the
screen must hand every row to the fp64 pass."""
import numpy as np
import pytest
import torch

import oracle
from parity import oracle_cfg, run_gpu, say
from vision_transformer_sparse_region_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    Workload("fp32_tie_attention_kernel", 2, 28, 28, 128, 4, 7, 4, "bf16", 136),
    Workload("fp32_tie_attention_argmax", 2, 56, 56, 64, 2, 7, 1, "bf16", 139),
    Workload("fp32_tie_attention_screened_topk", 2, 42, 42, 128, 4, 7, 4, "bf16", 142),
    Workload("fp32_tie_pool_route", 2, 14, 14, 256, 8, 7, 16, "bf16", 137),
    Workload("fp32_tie_route_large", 1, 40, 40, 64, 2, 10, 5, "bf16", 138),
]
A, B = 3, 5  # the two regions made best


def _inputs(wl):
    inp = make_inputs(wl)
    hs, ws = wl.height // wl.n_win, wl.width // wl.n_win
    q = (inp["q"].float() + 1.0).to(torch.bfloat16)
    k = inp["k"].clone()
    for reg, tweak in ((A, 0.0), (B, 2.0 ** -25)):
        ry, rx = divmod(reg, wl.n_win)
        tile = k[:, ry * hs:(ry + 1) * hs, rx * ws:(rx + 1) * ws, :]
        tile.fill_(4.0)
        # dim 0 of every head, first token: 0 in region A, 2^-25 in region B
        tile[:, 0, 0, ::32] = tweak
    inp["q"], inp["k"] = q.contiguous(), k.contiguous()
    return inp


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_routing_exact_where_fp32_keys_tie(wl):
    inp = _inputs(wl)
    say(f"[gpu] {wl.name}: B={wl.batch} {wl.height}x{wl.width} C={wl.channels} "
        f"heads={wl.num_heads} n_win={wl.n_win} topk={wl.topk}")
    _, gidx = run_gpu(wl, inp)
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v")}
    res = oracle.bra_forward(oracle_cfg(wl), f["q"], f["k"], f["v"], want_aff=True)
    aff = res["aff"]
    a, b = aff[..., A], aff[..., B]
    # the construction: distinct fp64 affinities that share an fp32 key, the
    # two best of the row
    assert (a != b).all()
    share = np.float32(a) == np.float32(b)
    assert share.mean() > 0.5, share.mean()
    if wl.topk >= 2:
        assert (np.sort(res["idx"][..., :2], axis=-1) == [A, B]).all()
    else:
        assert np.isin(res["idx"][..., 0], [A, B]).all()
    assert np.array_equal(gidx, res["idx"])


OVERFLOW = [
    Workload("fp32_overflow_argmax", 1, 56, 56, 64, 2, 7, 1, "bf16", 140),
    Workload("fp32_overflow_topk", 1, 56, 56, 64, 2, 7, 4, "bf16", 141),
]


@pytest.mark.parametrize("wl", OVERFLOW, ids=[w.name for w in OVERFLOW])
def test_routing_exact_where_fp32_products_overflow(wl):
    """Q and K scaled by 2^70: products of the means near 2^140 overflow fp32
    but not fp64.  Only the routing is compared (the attention scores overflow
    fp32 as well)."""
    inp = make_inputs(wl)
    scale = 2.0 ** 70
    inp["q"] = (inp["q"].float() * scale).to(torch.bfloat16)
    inp["k"] = (inp["k"].float() * scale).to(torch.bfloat16)
    say(f"[gpu] {wl.name}: B={wl.batch} {wl.height}x{wl.width} C={wl.channels} "
        f"heads={wl.num_heads} n_win={wl.n_win} topk={wl.topk}, q and k x 2^70")
    _, gidx = run_gpu(wl, inp)
    f = {n: inp[n].double().numpy() for n in ("q", "k", "v")}
    res = oracle.bra_forward(oracle_cfg(wl), f["q"], f["k"], f["v"], want_aff=True)
    assert np.isfinite(res["aff"]).all()
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.float32(res["aff"])).all()
    assert np.array_equal(gidx, res["idx"])
