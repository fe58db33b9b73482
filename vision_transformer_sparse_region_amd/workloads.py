"""Seeded synthetic workloads for the BRA forward pass.

This module only draws inputs; it holds none of the method's arithmetic, so
both the HIP path and the CPU oracle may be fed from it.

Shapes follow the stage table of "从零构建BiFormer：PyTorch实战双层路由注意力机制与调试全攻略"
(www.mhpn.cn/news/564882, §3: 56²/28²/14² maps, top-k 1/4/16, heads 2/4/8,
head_dim 32) and the 512x512 segmentation setting of
"BiFormer用双层路由注意力重塑视觉Transformer效率极限" (www.mooersco.com/news/894234,
§3.2) at stride 4 with the finer 16x16 region grid of its §4.1.  The datasets
those pages measure on are not used; these seeded tensors stand in for them.

Recipe (torch CPU generator seeded with `seed`, drawn in the order q, k, v,
lepe_w, lepe_b):
  * q, k, v: i.i.d. N(0, 1) in float32, rounded to bf16 (round-to-nearest-even)
    for bf16 workloads; for `smooth` workloads every (image, channel) plane is
    N(0, 1) noise blurred by a separable Gaussian (sigma 8 tokens, radius 32,
    reflect padding) and re-standardised to mean 0, std 1 before rounding, so
    that region affinities, and hence routing, depend on content.
  * lepe_w: [C, 5, 5] N(0, 0.02^2) float32.
  * lepe_b: zeros, or N(0, 0.02^2) when `lepe_bias` is set.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_proj_weights", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    height: int
    width: int
    channels: int
    num_heads: int
    n_win: int
    topk: int
    dtype: str  # "f32" or "bf16"
    seed: int
    smooth: bool = False
    lepe_bias: bool = False
    description: str = ""

    @property
    def head_dim(self) -> int:
        return self.channels // self.num_heads

    @property
    def regions(self) -> int:
        return self.n_win * self.n_win

    @property
    def tokens_per_region(self) -> int:
        return (self.height // self.n_win) * (self.width // self.n_win)

    @property
    def topk_effective(self) -> int:
        r = self.regions
        return r if self.topk <= 0 or self.topk > r else self.topk

    @property
    def tokens(self) -> int:
        return self.batch * self.height * self.width

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 1, 28, 28, 64, 2, 7, 4, "f32", 1,
        description="tiny fp32 BRA: B=1, 28x28, n_win=7 (49 regions of 4x4), 2 heads x 32, topk=4"),
    "stage1": Workload(
        "stage1", 64, 56, 56, 64, 2, 7, 1, "bf16", 2,
        description="BiFormer-S stage-1 BRA: B=64, 56x56, n_win=7 (49 regions of 8x8), "
                    "2 heads x 32, topk=1, bf16"),
    "stage2": Workload(
        "stage2", 64, 28, 28, 128, 4, 7, 4, "bf16", 3,
        description="BiFormer-S stage-2 BRA: B=64, 28x28, n_win=7 (49 regions of 4x4), "
                    "4 heads x 32, topk=4, bf16"),
    "stage3": Workload(
        "stage3", 64, 14, 14, 256, 8, 7, 16, "bf16", 4,
        description="BiFormer-S stage-3 BRA: B=64, 14x14, n_win=7 (49 regions of 2x2), "
                    "8 heads x 32, topk=16, bf16"),
    "highres": Workload(
        "highres", 8, 128, 128, 64, 2, 16, 16, "bf16", 5, smooth=True,
        description="512x512 segmentation at stride 4 BRA: B=8, 128x128, n_win=16 "
                    "(256 regions of 8x8), 2 heads x 32, topk=16, bf16, smooth fields"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _gauss_blur_planes(x: torch.Tensor, sigma: float) -> torch.Tensor:
    """Separable Gaussian blur of every [H, W] plane of x [P, H, W] (reflect pad)."""
    radius = int(4 * sigma)
    taps = torch.arange(-radius, radius + 1, dtype=torch.float32)
    g = torch.exp(-0.5 * (taps / sigma) ** 2)
    g = g / g.sum()
    p, h, w = x.shape
    y = x.reshape(p * h, 1, w)
    y = torch.nn.functional.pad(y, (radius, radius), mode="reflect")
    y = torch.nn.functional.conv1d(y, g.view(1, 1, -1)).reshape(p, h, w)
    y = y.transpose(1, 2).reshape(p * w, 1, h)
    y = torch.nn.functional.pad(y, (radius, radius), mode="reflect")
    y = torch.nn.functional.conv1d(y, g.view(1, 1, -1)).reshape(p, w, h).transpose(1, 2)
    return y


def _draw_map(gen: torch.Generator, wl: Workload) -> torch.Tensor:
    shape = (wl.batch, wl.height, wl.width, wl.channels)
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if wl.smooth:
        planes = x.permute(0, 3, 1, 2).reshape(wl.batch * wl.channels, wl.height, wl.width)
        planes = _gauss_blur_planes(planes, 8.0)
        mean = planes.mean(dim=(1, 2), keepdim=True)
        std = planes.std(dim=(1, 2), keepdim=True)
        planes = (planes - mean) / std
        x = planes.reshape(wl.batch, wl.channels, wl.height, wl.width).permute(0, 2, 3, 1)
        x = x.contiguous()
    return x.to(wl.torch_dtype)


def make_inputs(wl: Workload) -> dict:
    """Return CPU tensors q, k, v ([B,H,W,C], wl dtype), lepe_w [C,5,5], lepe_b [C] (fp32)."""
    gen = torch.Generator().manual_seed(wl.seed)
    q = _draw_map(gen, wl)
    k = _draw_map(gen, wl)
    v = _draw_map(gen, wl)
    lepe_w = torch.randn((wl.channels, 5, 5), generator=gen, dtype=torch.float32) * 0.02
    if wl.lepe_bias:
        lepe_b = torch.randn((wl.channels,), generator=gen, dtype=torch.float32) * 0.02
    else:
        lepe_b = torch.zeros((wl.channels,), dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "lepe_w": lepe_w, "lepe_b": lepe_b}


def make_proj_weights(wl: Workload, seed: int | None = None) -> dict:
    """Random Linear weights of the module's projections (bf16, PyTorch [out, in]
    layout) and fp32 biases, drawn in the order w_qkv, b_qkv, w_o, b_o from a
    generator seeded with `seed` (default wl.seed + 1000): w ~ N(0, 1/C), so
    a projection of N(0, 1) inputs has unit variance, and b ~ N(0, 0.02^2).
    Synthetic stand-ins for trained weights; the draws only."""
    gen = torch.Generator().manual_seed(wl.seed + 1000 if seed is None else seed)
    C = wl.channels
    std = C ** -0.5
    w_qkv = (torch.randn((3 * C, C), generator=gen) * std).to(torch.bfloat16)
    b_qkv = torch.randn((3 * C,), generator=gen) * 0.02
    w_o = (torch.randn((C, C), generator=gen) * std).to(torch.bfloat16)
    b_o = torch.randn((C,), generator=gen) * 0.02
    return {"w_qkv": w_qkv, "b_qkv": b_qkv, "w_o": w_o, "b_o": b_o}
