"""GPU: the forward captured in a HIP graph and replayed.

The entry points only enqueue kernels on the caller's stream (no allocation,
no synchronisation, no memset), so a caller can capture them.  Each replay
must reproduce the eager result bit for bit (the kernels are deterministic),
with eager work and synchronisations between the replays, as a graph is used
in practice.
"""
import pytest
import torch

from parity import say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import (WORKLOADS, make_inputs,
                                                           make_proj_weights)

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_replays(g, outs, refs):
    for rep in range(REPLAYS):
        for t in outs:
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t,
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r), rep


@pytest.mark.parametrize("name", ["stage1", "stage3", "highres", "tiny_f32"])
def test_forward_graph_replays_match_eager(name):
    wl = WORKLOADS[name]
    wl = wl.with_(batch=min(wl.batch, 2))
    dev = torch.device("cuda:0")
    inp = {n: t.to(dev) for n, t in make_inputs(wl).items()}
    say(f"[gpu] graph replay: {wl.name} B={wl.batch}")
    with bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                 wl.dtype) as h:
        ref, ref_idx = h.forward(inp["q"], inp["k"], inp["v"], inp["lepe_w"], inp["lepe_b"])
        torch.cuda.synchronize()
        out, idx = torch.empty_like(ref), torch.empty_like(ref_idx)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            h.forward(inp["q"], inp["k"], inp["v"], inp["lepe_w"], inp["lepe_b"], out=out,
                      routing_idx=idx)
        _check_replays(g, [out, idx], [ref, ref_idx])


@pytest.mark.parametrize("name", ["stage1", "stage3"])
def test_projected_forward_graph_replays_match_eager(name):
    """Both places of the output projection: the attention epilogue (stage
    1) and its own kernel (stage 3)."""
    wl = WORKLOADS[name].with_(batch=2)
    dev = torch.device("cuda:0")
    inp = {n: t.to(dev) for n, t in make_inputs(wl).items()}
    w = {n: t.to(dev) for n, t in make_proj_weights(wl).items()}
    say(f"[gpu] graph replay, projections: {wl.name} B={wl.batch}")
    with bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                 wl.dtype, projections=True) as h:
        args = (inp["q"], w["w_qkv"], w["w_o"], w["b_qkv"], w["b_o"], inp["lepe_w"],
                inp["lepe_b"])
        ref, ref_idx = h.forward_proj(*args)
        torch.cuda.synchronize()
        out, idx = torch.empty_like(ref), torch.empty_like(ref_idx)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            h.forward_proj(*args, out=out, routing_idx=idx)
        _check_replays(g, [out, idx], [ref, ref_idx])
