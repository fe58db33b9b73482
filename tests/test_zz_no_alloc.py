"""GPU: the allocation-free forward (bra_forward_noalloc, for callers that
cannot allocate) against bra_forward through the C ABI.  The two share every
kernel; only the workspace differs (the library's device scratch array
instead of the handle's allocation), so their outputs and routings must be
identical -- which also meets the parity bar of tests/parity.py.  Two calls
in a row, the second on a smaller input, then the other paths the
workspace serves: the image kernel with the routing kept in scratch, the
routing kernel over 256 regions, and the zero bias that a missing lepe_b
stands for."""
import numpy as np
import pytest
import torch

from parity import TOL, max_rel_err, say
from vision_transformer_sparse_region_amd import bra
from vision_transformer_sparse_region_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _both(wl, bias=True, want_idx=True):
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    w = inp["lepe_w"].to(dev)
    b = inp["lepe_b"].to(dev) if bias else None
    with bra.BRA(wl.batch, wl.height, wl.width, wl.channels, wl.num_heads, wl.n_win, wl.topk,
                 wl.dtype) as h:
        ref, ref_idx = h.forward(q, k, v, w, b, routing_idx=want_idx)
        cfg = h.cfg
    out = torch.empty_like(q)
    idx = torch.empty_like(ref_idx) if want_idx else None
    bra.bra_forward_noalloc(cfg, q, k, v, w, b, out, idx)
    torch.cuda.synchronize()
    return ref, ref_idx, out, idx


@pytest.mark.parametrize("wl", [WORKLOADS["stage1"].with_(batch=4, seed=501),
                                WORKLOADS["stage1"].with_(batch=2, seed=502)],
                         ids=["first_call_b4", "second_call_b2"])
def test_noalloc_equals_forward_two_calls(wl):
    say(f"[gpu] noalloc {wl.name} B={wl.batch}")
    ref, ref_idx, out, idx = _both(wl)
    assert torch.equal(idx, ref_idx)
    err = max_rel_err(out.cpu(), ref.cpu().double().numpy(), wl.num_heads)
    assert err <= TOL[wl.dtype]
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("wl,bias,want_idx", [
    (WORKLOADS["stage3"].with_(batch=2, seed=503), True, False),
    (WORKLOADS["highres"].with_(batch=1, seed=504), True, True),
    (WORKLOADS["stage1"].with_(batch=1, seed=505), False, True),
], ids=["image_kernel_routing_in_scratch", "routing_kernel", "zero_bias"])
def test_noalloc_other_paths(wl, bias, want_idx):
    say(f"[gpu] noalloc {wl.name} B={wl.batch} bias={bias} idx={want_idx}")
    ref, ref_idx, out, idx = _both(wl, bias=bias, want_idx=want_idx)
    if want_idx:
        assert torch.equal(idx, ref_idx)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
