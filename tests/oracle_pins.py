"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises ``AssertionError`` when
the oracle disagrees with what the pages and the mathematics fix:

* closed forms and special cases that reduce to a library routine (dense
  softmax attention when every region is routed, one region per map, constant
  V, all-zero K, a depthwise convolution),
* brute force on tiny inputs (argsort of an affinity computed with numpy
  window reshapes),
* invariants (positive scaling of q, permutation of the routed set),
* forced exact ties, a hand-worked example, and an independent PyTorch
  formulation built from library gather/topk/softmax/conv2d calls.

``tests/test_oracle_pins.py`` runs them against the real oracle and
``tests/test_oracle_mutants.py`` against deliberately broken builds, each of
which at least one pin must reject.

Page keys: [P1] www.mhpn.cn/news/199372, [P2] www.mooersco.com/news/894234,
[P3] www.mhpn.cn/news/564882, [P4] www.jsqmd.com/news/719213,
[P5] www.mhpn.cn/news/2512273.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import OracleConfig

RTOL = 1e-10
ATOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_map(rng, cfg, scale=1.0):
    return rng.standard_normal((cfg.batch, cfg.height, cfg.width, cfg.channels)) * scale


def _rand_lepe(rng, cfg, bias=True):
    w = rng.standard_normal((cfg.channels, 5, 5)) * 0.02
    b = rng.standard_normal((cfg.channels,)) * 0.02 if bias else None
    return w, b


# ---- independent library formulations ------------------------------------

def np_windows(x, n):
    """[B,H,W,C] -> [B, R, t, C] with square windows, row-major inside.  [P3 §1]"""
    B, H, W, C = x.shape
    hs, ws = H // n, W // n
    return x.reshape(B, n, hs, n, ws, C).transpose(0, 1, 3, 2, 4, 5).reshape(B, n * n, hs * ws, C)


def np_unwindows(xw, n, H, W):
    B, R, t, C = xw.shape
    hs, ws = H // n, W // n
    return xw.reshape(B, n, n, hs, ws, C).transpose(0, 1, 3, 2, 4, 5).reshape(B, H, W, C)


def np_head_means(x, n, heads):
    """Per-head region means [B, h, R, hd] via numpy mean over window tokens."""
    xw = np_windows(x, n)
    B, R, t, C = xw.shape
    m = xw.mean(axis=2).reshape(B, R, heads, C // heads)
    return m.transpose(0, 2, 1, 3)


def torch_dense_attention(q, k, v, heads, scale=None):
    """softmax(q k^T * scale) v over all tokens of each image, per head (library SDPA)."""
    B, H, W, C = q.shape
    hd = C // heads

    def split(x):
        return torch.from_numpy(np.ascontiguousarray(x)).reshape(B, H * W, heads, hd).permute(0, 2, 1, 3)

    o = torch.nn.functional.scaled_dot_product_attention(split(q), split(k), split(v),
                                                         scale=scale)
    return o.permute(0, 2, 1, 3).reshape(B, H, W, C).numpy()


def torch_lepe(v, w, b):
    """Depthwise Conv2d(C, C, 5, padding=2, groups=C) in float64.  [P5 §五 self.lepe]"""
    C = v.shape[-1]
    x = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(np.ascontiguousarray(w)).reshape(C, 1, 5, 5)
    bt = torch.from_numpy(np.ascontiguousarray(b)) if b is not None else None
    y = torch.nn.functional.conv2d(x, wt, bt, padding=2, groups=C)
    return y.permute(0, 2, 3, 1).numpy()


def torch_bra_recipe(cfg: OracleConfig, q, k, v, w, b, shared=False):
    """The pages' PyTorch recipe in float64: window partition [P3 §1], per-head
    means and affinity [P5 §五 ③], torch.topk [P5 §五 ④], torch.gather of the
    routed windows [P5 §五 ⑤], softmax attention [P5 §五 ⑥], LePE of V added.
    shared=True routes with the full-C means, one index for every head, as
    P2 §2.1 and P3 §2.1 do (their affinity is [B, R, R])."""
    B, H, W, C = q.shape
    n, h = cfg.n_win, cfg.num_heads
    hd = C // h
    R = n * n
    k_eff = R if cfg.topk <= 0 or cfg.topk > R else cfg.topk
    scale = cfg.scale if cfg.scale > 0 else hd ** -0.5

    def regions(x):  # [B, h, R, t, hd]
        xw = torch.from_numpy(np_windows(x, n))
        t = xw.shape[2]
        return xw.reshape(B, R, t, h, hd).permute(0, 3, 1, 2, 4)

    qr, kr, vr = regions(q), regions(k), regions(v)
    t = qr.shape[3]
    if shared:
        # full-C region means [B, R, C] from the unsplit windows
        qf = torch.from_numpy(np_windows(q, n)).mean(dim=2)
        kf = torch.from_numpy(np_windows(k, n)).mean(dim=2)
        sidx = (qf @ kf.transpose(-1, -2)).topk(k_eff, dim=-1).indices  # [B, R, k]
        idx = sidx.unsqueeze(1).expand(B, h, R, k_eff)
    else:
        aff = qr.mean(dim=3) @ kr.mean(dim=3).transpose(-1, -2)
        idx = aff.topk(k_eff, dim=-1).indices  # [B, h, R, k]

    def gather(x):
        xe = x.unsqueeze(2).expand(B, h, R, R, t, hd)
        ie = idx[..., None, None].expand(B, h, R, k_eff, t, hd)
        return torch.gather(xe, 3, ie).reshape(B, h, R, k_eff * t, hd)

    kg, vg = gather(kr), gather(vr)
    attn = torch.softmax((qr * scale) @ kg.transpose(-1, -2), dim=-1)
    o = attn @ vg  # [B, h, R, t, hd]
    o = o.permute(0, 2, 3, 1, 4).reshape(B, R, t, C).numpy()
    out = np_unwindows(o, n, H, W)
    if w is not None:
        out = out + torch_lepe(v, w, b)
    idx = sidx if shared else idx
    return out, idx.numpy().astype(np.int32)


# ---- pins ----------------------------------------------------------------

def pin_topk_all_is_dense_attention(orc):
    """Routing every region to every region is dense attention over the map."""
    for (B, H, W, heads, hd, n, topk, scale) in [
        (2, 8, 12, 2, 8, 2, -1, 0.0),
        (1, 6, 6, 3, 4, 3, 9, 0.0),
        (1, 8, 8, 1, 32, 4, 1000, 0.3),
    ]:
        cfg = OracleConfig(B, H, W, heads * hd, heads, n, topk, scale)
        rng = _rng(H * 100 + W)
        q, k, v = (_rand_map(rng, cfg) for _ in range(3))
        res = orc.bra_forward(cfg, q, k, v)
        ref = torch_dense_attention(q, k, v, heads, scale if scale > 0 else None)
        np.testing.assert_allclose(res["out"], ref, rtol=RTOL, atol=ATOL)
        # every row of the routing is a permutation of all regions
        R = n * n
        assert res["idx"].shape[-1] == R
        assert (np.sort(res["idx"], axis=-1) == np.arange(R)).all()


def pin_one_region_is_dense_attention(orc):
    """n_win = 1: one region, k = 1, again dense attention."""
    cfg = OracleConfig(2, 6, 10, 16, 2, 1, 1)
    rng = _rng(7)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    res = orc.bra_forward(cfg, q, k, v)
    np.testing.assert_allclose(res["out"], torch_dense_attention(q, k, v, 2),
                               rtol=RTOL, atol=ATOL)
    assert (res["idx"] == 0).all()


def pin_constant_v(orc):
    """Softmax weights sum to one: V constant over the map returns that
    constant; with LePE the border-aware sum of in-map taps is added."""
    cfg = OracleConfig(2, 8, 8, 8, 2, 2, 2)
    rng = _rng(11)
    q, k = _rand_map(rng, cfg), _rand_map(rng, cfg)
    c = rng.standard_normal(cfg.channels)
    v = np.broadcast_to(c, (2, 8, 8, 8)).copy()
    res = orc.bra_forward(cfg, q, k, v)
    np.testing.assert_allclose(res["out"], v, rtol=0, atol=1e-12)
    w, b = _rand_lepe(rng, cfg)
    res = orc.bra_forward(cfg, q, k, v, w, b)
    # in-map tap mask: tap (i, j) at (y, x) reads (y+i-2, x+j-2)
    ys = np.arange(8)[:, None] + np.arange(5)[None, :] - 2
    valid_y = (ys >= 0) & (ys < 8)  # [y, i]
    tapmask = valid_y[:, None, :, None] & valid_y[None, :, None, :]  # [y, x, i, j]
    wsum = np.einsum("yxij,cij->yxc", tapmask.astype(np.float64), w)
    expect = c * (1.0 + wsum) + b
    np.testing.assert_allclose(res["out"], np.broadcast_to(expect, v.shape), rtol=0, atol=1e-12)


def pin_zero_k_uniform_over_lowest_regions(orc):
    """K = 0 makes every affinity 0 (all tied, so regions 0..k-1 are routed)
    and every logit 0 (uniform softmax): the output is the plain mean of V
    over the tokens of regions 0..k-1."""
    cfg = OracleConfig(2, 8, 12, 8, 2, 2, 3)
    rng = _rng(13)
    q, v = _rand_map(rng, cfg), _rand_map(rng, cfg)
    k = np.zeros_like(q)
    res = orc.bra_forward(cfg, q, k, v)
    assert (res["idx"] == np.arange(3)).all()
    vw = np_windows(v, 2)  # [B, R, t, C]
    mean_lowest = vw[:, :3].reshape(2, -1, 8).mean(axis=1)  # [B, C]
    np.testing.assert_allclose(res["out"], np.broadcast_to(mean_lowest[:, None, None, :],
                                                           v.shape), rtol=RTOL, atol=ATOL)


def pin_means_match_numpy(orc):
    """Per-head window means equal numpy's mean over the reshaped windows."""
    cfg = OracleConfig(2, 12, 8, 12, 3, 4, 2)
    rng = _rng(17)
    x = _rand_map(rng, cfg)
    np.testing.assert_allclose(orc.region_means(cfg, x), np_head_means(x, 4, 3),
                               rtol=1e-13, atol=1e-15)


def pin_region_sums_exact_within_span(orc):
    """Region sums of bf16 values [P4 §1.2; P5 §五 ③].  The nonzero values of one
    (region, channel) are multiples of the smallest one's last significand
    bit; while they span at most 2^(45 - ceil(log2 t)) in magnitude every
    partial sum is an integer below 2^53 of those units, so every order of
    the additions gives the exact sum (math.fsum) -- the fact that lets the
    kernels sum as trees.  Here t = 64 and the span 2^39: the oracle's mean
    is fsum / t to the last bit, and so is a pairwise tree.  Past the span
    the orders differ, and the oracle keeps the slot order: 1 + 1 + 2^60 -
    2^60 is 0 summed left to right, 2 summed as a tree."""
    cfg = OracleConfig(1, 8, 8, 32, 1, 1, 1)  # one region of 64 tokens
    rng = _rng(29)
    e = rng.integers(-20, 20, size=(1, 8, 8, 32))  # exponents span 39 binades
    sig = rng.integers(128, 256, size=e.shape) * rng.choice([-1, 1], size=e.shape)
    x = sig * np.exp2(e - 7.0)  # 8-bit significands: exact bf16 values
    means = orc.region_means(cfg, x)[0, 0, 0]
    for c in range(32):
        col = x[0, :, :, c].reshape(-1)  # slot order = row-major in the window
        exact = math.fsum(col.tolist())
        tree = col.copy()
        while tree.size > 1:
            tree = tree[0::2] + tree[1::2]
        assert tree[0] == exact, c
        assert means[c] == exact / 64, (c, means[c], exact / 64)
    y = np.zeros((1, 8, 8, 32))
    y[0, 0, :4, 0] = [1.0, 1.0, 2.0 ** 60, -(2.0 ** 60)]
    col = y[0, :, :, 0].reshape(-1)
    tree = col.copy()
    while tree.size > 1:
        tree = tree[0::2] + tree[1::2]
    assert tree[0] == 2.0 and math.fsum(col.tolist()) == 2.0
    assert orc.region_means(cfg, y)[0, 0, 0, 0] == 0.0


def pin_routing_bruteforce_argsort(orc):
    """Routing equals a stable argsort of an independently computed affinity."""
    for (B, H, W, heads, hd, n, topk, seed) in [
        (2, 12, 8, 2, 8, 4, 5, 19), (1, 14, 14, 1, 32, 7, 4, 23), (3, 6, 9, 3, 4, 3, 9, 29)]:
        cfg = OracleConfig(B, H, W, heads * hd, heads, n, topk)
        rng = _rng(seed)
        q, k = _rand_map(rng, cfg), _rand_map(rng, cfg)
        res = orc.bra_forward(cfg, q, k, _rand_map(rng, cfg), want_aff=True, want_means=True)
        qb, kb = np_head_means(q, n, heads), np_head_means(k, n, heads)
        aff = np.einsum("bhrd,bhsd->bhrs", qb, kb)
        np.testing.assert_allclose(res["aff"], aff, rtol=1e-12, atol=1e-14)
        k_eff = min(topk, n * n) if topk > 0 else n * n
        expect = np.argsort(-aff, axis=-1, kind="stable")[..., :k_eff]
        assert (res["idx"] == expect).all()


def pin_ties_go_to_lower_region(orc):
    """Exact ties are broken toward the lower region id."""
    cfg = OracleConfig(1, 8, 8, 8, 2, 4, 5)
    rng = _rng(31)
    q = _rand_map(rng, cfg)
    # (a) every region of K identical -> every affinity in a row equal
    tile = rng.standard_normal((2, 2, 8))
    k = np.tile(tile, (4, 4, 1))[None]
    res = orc.bra_forward(cfg, q, k, _rand_map(rng, cfg))
    assert (res["idx"] == np.arange(5)).all()
    # (b) region 2 and region 9 of K identical -> exact tie between 2 and 9
    k = _rand_map(rng, cfg)
    kw = np_windows(k, 4)
    kw[:, 9] = kw[:, 2]
    k = np_unwindows(kw, 4, 8, 8)
    cfg16 = OracleConfig(1, 8, 8, 8, 2, 4, 16)
    res = orc.bra_forward(cfg16, q, k, k)
    for row in res["idx"].reshape(-1, 16):
        pos = {int(s): j for j, s in enumerate(row)}
        assert pos[9] == pos[2] + 1, row


def pin_positive_scaling_keeps_routing(orc):
    """Scaling q by a positive constant scales every affinity: routing unchanged."""
    cfg = OracleConfig(2, 12, 12, 16, 2, 3, 4)
    rng = _rng(37)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    base = orc.bra_forward(cfg, q, k, v)["idx"]
    for a in (3.0, 0.37, 1e3):
        assert (orc.bra_forward(cfg, q * a, k, v)["idx"] == base).all()


def pin_routed_set_order_free(orc):
    """Attention over the routed set does not depend on the order of its ids."""
    cfg = OracleConfig(2, 8, 8, 8, 2, 4, 4)
    rng = _rng(41)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    idx = orc.bra_forward(cfg, q, k, v)["idx"]
    perm = np.ascontiguousarray(idx[..., ::-1])
    np.testing.assert_allclose(orc.attend(cfg, q, k, v, perm), orc.attend(cfg, q, k, v, idx),
                               rtol=RTOL, atol=ATOL)


def pin_lepe_matches_conv2d(orc):
    """LePE equals the library depthwise convolution (zero padding 2, bias)."""
    cfg = OracleConfig(2, 7, 9, 6, 2, 1, 1)
    rng = _rng(43)
    v = _rand_map(rng, cfg)
    w, b = _rand_lepe(rng, cfg)
    np.testing.assert_allclose(orc.lepe(cfg, v, w, b), torch_lepe(v, w, b), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(orc.lepe(cfg, v, w, None), torch_lepe(v, w, None), rtol=1e-12,
                               atol=1e-14)


def pin_lepe_impulse_orientation(orc):
    """A unit impulse at (y0, x0) puts tap (i, j) at (y0+2-i, x0+2-j) (the
    cross-correlation orientation of Conv2d), e.g. w[3, 2] at (y0-1, x0)."""
    cfg = OracleConfig(1, 9, 9, 2, 1, 1, 1)
    rng = _rng(47)
    w, _ = _rand_lepe(rng, cfg, bias=False)
    v = np.zeros((1, 9, 9, 2))
    v[0, 4, 4, 1] = 1.0
    L = orc.lepe(cfg, v, w, None)
    assert L[0, 3, 4, 1] == w[1, 3, 2]
    for i in range(5):
        for j in range(5):
            assert L[0, 4 + 2 - i, 4 + 2 - j, 1] == w[1, i, j]
    assert (L[..., 0] == 0).all()


def pin_hand_worked_single_token_regions(orc):
    """A 2x2 map with n_win = 2 has one token per region, so the region means
    are the tokens and the affinity is q_p . k_s.  Worked by hand:
      q = (1,0), (0,1), (-1,0), (0,-1);  k = (1,0), (0,1), (0,0), (2,2)
      rows of A: [1,0,0,2], [0,1,0,2], [-1,0,0,-2], [0,-1,0,-2]
      top-1: 3, 3, 1 (tie 1|2 -> 1), 0 (tie 0|2 -> 0); one key each, so out = v[idx].
      top-2 of row 0 is (3, 0); the logits are 2s and 1s with s = 2^-0.5, so
      out_0 = (e^{2s} v_3 + e^{s} v_0) / (e^{2s} + e^{s})."""
    q = np.array([[1, 0], [0, 1], [-1, 0], [0, -1]], np.float64).reshape(1, 2, 2, 2)
    k = np.array([[1, 0], [0, 1], [0, 0], [2, 2]], np.float64).reshape(1, 2, 2, 2)
    v = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], np.float64).reshape(1, 2, 2, 2)
    cfg = OracleConfig(1, 2, 2, 2, 1, 2, 1)
    res = orc.bra_forward(cfg, q, k, v)
    assert res["idx"].reshape(-1).tolist() == [3, 3, 1, 0]
    np.testing.assert_array_equal(res["out"].reshape(4, 2), v.reshape(4, 2)[[3, 3, 1, 0]])
    cfg2 = OracleConfig(1, 2, 2, 2, 1, 2, 2)
    res = orc.bra_forward(cfg2, q, k, v)
    assert res["idx"][0, 0, 0].tolist() == [3, 0]
    s = 2 ** -0.5
    e2, e1 = math.exp(2 * s), math.exp(s)
    expect0 = (e2 * np.array([7.0, 8.0]) + e1 * np.array([1.0, 2.0])) / (e2 + e1)
    np.testing.assert_allclose(res["out"][0, 0, 0], expect0, rtol=1e-14)


def pin_matches_torch_recipe(orc):
    """The whole forward equals the pages' PyTorch recipe in float64."""
    for (B, H, W, heads, hd, n, topk, seed) in [
        (2, 8, 8, 2, 8, 2, 2, 53), (1, 12, 16, 2, 32, 4, 3, 59), (2, 9, 6, 3, 4, 3, 4, 61)]:
        cfg = OracleConfig(B, H, W, heads * hd, heads, n, topk)
        rng = _rng(seed)
        q, k, v = (_rand_map(rng, cfg) for _ in range(3))
        w, b = _rand_lepe(rng, cfg)
        res = orc.bra_forward(cfg, q, k, v, w, b)
        ref_out, ref_idx = torch_bra_recipe(cfg, q, k, v, w, b)
        assert (res["idx"] == ref_idx).all()
        np.testing.assert_allclose(res["out"], ref_out, rtol=RTOL, atol=ATOL)


def pin_lepe_reads_v(orc):
    """The LePE term is a convolution of V (not of q, k or the attention
    output): with q = k = 0 the forward is mean(V) plus conv(V)."""
    cfg = OracleConfig(1, 8, 8, 4, 1, 2, 4)
    rng = _rng(67)
    v = _rand_map(rng, cfg)
    w, b = _rand_lepe(rng, cfg)
    z = np.zeros_like(v)
    res = orc.bra_forward(cfg, z, z, v, w, b)
    mean = v.reshape(-1, 4).mean(axis=0)
    np.testing.assert_allclose(res["out"], mean + torch_lepe(v, w, b), rtol=RTOL, atol=ATOL)


def pin_topk_clamp(orc):
    """k actually used: min(topk, R), topk <= 0 meaning all regions."""
    for topk, expect in [(-1, 16), (0, 16), (16, 16), (40, 16), (1, 1), (7, 7)]:
        assert orc.topk_effective(OracleConfig(1, 8, 8, 4, 1, 4, topk)) == expect


# ---- head-shared routing [P1 §2.2; P2 §2.1; P3 §2.1; P4 §1.2] --------------

def pin_shared_routing_bruteforce_argsort(orc):
    """Head-shared routing equals a stable argsort of the affinity of the
    full-C window means, computed with numpy reshapes."""
    for (B, H, W, heads, hd, n, topk, seed) in [
        (2, 12, 8, 2, 8, 4, 5, 71), (1, 14, 14, 4, 8, 7, 4, 73), (3, 6, 9, 3, 4, 3, 9, 79)]:
        cfg = OracleConfig(B, H, W, heads * hd, heads, n, topk)
        rng = _rng(seed)
        q, k = _rand_map(rng, cfg), _rand_map(rng, cfg)
        res = orc.bra_forward_shared(cfg, q, k, _rand_map(rng, cfg), want_aff=True)
        qf, kf = np_windows(q, n).mean(axis=2), np_windows(k, n).mean(axis=2)
        aff = np.einsum("brc,bsc->brs", qf, kf)
        np.testing.assert_allclose(res["aff"], aff, rtol=1e-12, atol=1e-14)
        k_eff = min(topk, n * n) if topk > 0 else n * n
        expect = np.argsort(-aff, axis=-1, kind="stable")[..., :k_eff]
        assert (res["idx"] == expect).all()


def pin_shared_routing_one_head_is_per_head(orc):
    """With one head, head-shared and per-head routing coincide (bit for bit)."""
    cfg = OracleConfig(2, 12, 12, 16, 1, 3, 4)
    rng = _rng(83)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    w, b = _rand_lepe(rng, cfg)
    per = orc.bra_forward(cfg, q, k, v, w, b, want_aff=True)
    sh = orc.bra_forward_shared(cfg, q, k, v, w, b, want_aff=True)
    assert (sh["idx"] == per["idx"][:, 0]).all()
    np.testing.assert_array_equal(sh["aff"], per["aff"][:, 0])
    np.testing.assert_array_equal(sh["out"], per["out"])


def pin_shared_routing_sums_head_affinities(orc):
    """The shared affinity is the sum of the per-head affinities (to rounding),
    and every head attends over the shared routed set."""
    cfg = OracleConfig(2, 8, 8, 12, 3, 4, 3)
    rng = _rng(89)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    per = orc.bra_forward(cfg, q, k, v, want_aff=True)
    sh = orc.bra_forward_shared(cfg, q, k, v, want_aff=True)
    np.testing.assert_allclose(sh["aff"], per["aff"].sum(axis=1), rtol=1e-12, atol=1e-13)
    full = np.ascontiguousarray(np.repeat(sh["idx"][:, None], 3, axis=1))
    np.testing.assert_allclose(sh["out"], orc.attend(cfg, q, k, v, full), rtol=RTOL, atol=ATOL)


def pin_shared_ties_go_to_lower_region(orc):
    """Exact ties in the shared affinity go to the lower region id."""
    cfg = OracleConfig(1, 8, 8, 8, 2, 4, 5)
    rng = _rng(97)
    q = _rand_map(rng, cfg)
    tile = rng.standard_normal((2, 2, 8))
    k = np.tile(tile, (4, 4, 1))[None]
    res = orc.bra_forward_shared(cfg, q, k, _rand_map(rng, cfg))
    assert (res["idx"] == np.arange(5)).all()


def pin_shared_matches_torch_recipe(orc):
    """The whole forward with head-shared routing equals the pages' PyTorch
    recipe with full-C routing, in float64."""
    for (B, H, W, heads, hd, n, topk, seed) in [
        (2, 8, 8, 2, 8, 2, 2, 101), (1, 12, 16, 4, 8, 4, 3, 103), (2, 9, 6, 3, 4, 3, 4, 107)]:
        cfg = OracleConfig(B, H, W, heads * hd, heads, n, topk)
        rng = _rng(seed)
        q, k, v = (_rand_map(rng, cfg) for _ in range(3))
        w, b = _rand_lepe(rng, cfg)
        res = orc.bra_forward_shared(cfg, q, k, v, w, b)
        ref_out, ref_idx = torch_bra_recipe(cfg, q, k, v, w, b, shared=True)
        assert (res["idx"] == ref_idx).all()
        np.testing.assert_allclose(res["out"], ref_out, rtol=RTOL, atol=ATOL)


# ---- KV downsampling [P1 §4.1 kv_downsample_ratio, avgpool] ----------------

def torch_avg_pool(x, ratio):
    """[B,H,W,C] average-pooled over ratio x ratio blocks (library avg_pool2d)."""
    xt = torch.from_numpy(np.ascontiguousarray(x)).permute(0, 3, 1, 2)
    return torch.nn.functional.avg_pool2d(xt, ratio).permute(0, 2, 3, 1).numpy()


def pin_kv_downsample_matches_avg_pool(orc):
    """The downsampled K/V equal the library's average pooling."""
    cfg = OracleConfig(2, 16, 8, 6, 2, 2, 1)
    rng = _rng(109)
    x = _rand_map(rng, cfg)
    for ratio in (1, 2, 4):
        np.testing.assert_allclose(orc.kv_downsample(cfg, ratio, x), torch_avg_pool(x, ratio),
                                   rtol=1e-13, atol=1e-15)
    # a ratio that does not divide the window sides is refused
    try:
        orc.kv_downsample(cfg, 3, x)
    except ValueError:
        pass
    else:
        raise AssertionError("ratio 3 accepted for 8x4 windows")


def pin_kvds_ratio_one_is_plain(orc):
    """Ratio 1 is the plain forward, bit for bit."""
    cfg = OracleConfig(2, 8, 8, 16, 2, 2, 2)
    rng = _rng(113)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    w, b = _rand_lepe(rng, cfg)
    a = orc.bra_forward(cfg, q, k, v, w, b)
    d = orc.bra_forward_kvds(cfg, 1, q, k, v, w, b)
    assert (a["idx"] == d["idx"]).all()
    np.testing.assert_array_equal(a["out"], d["out"])


def pin_kvds_all_regions_is_dense_over_pooled(orc):
    """Every region routed: each query attends to the whole downsampled map --
    dense attention (library SDPA) over avg-pooled K and V -- plus the LePE of
    the full-resolution V."""
    cfg = OracleConfig(2, 8, 8, 16, 2, 2, 4)
    rng = _rng(127)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    w, b = _rand_lepe(rng, cfg)
    for ratio in (2, 4):
        kd, vd = torch_avg_pool(k, ratio), torch_avg_pool(v, ratio)
        B, H, W, C = q.shape
        hd = C // 2

        def heads(x):
            n = x.shape[1] * x.shape[2]
            return torch.from_numpy(np.ascontiguousarray(x)).reshape(B, n, 2, hd).permute(0, 2, 1, 3)

        o = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(kd), heads(vd))
        o = o.permute(0, 2, 1, 3).reshape(B, H, W, C).numpy()
        res = orc.bra_forward_kvds(cfg, ratio, q, k, v, w, b)
        np.testing.assert_allclose(res["out"], o + torch_lepe(v, w, b), rtol=RTOL, atol=ATOL)


def pin_attend_kvds_matches_forward(orc):
    """Attention over the downsampled K/V with the forward's own routing, plus
    LePE, is the KV-downsampled forward; ratio 1 is the plain attention."""
    cfg = OracleConfig(2, 8, 8, 16, 2, 2, 2)
    rng = _rng(137)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    w, b = _rand_lepe(rng, cfg)
    res = orc.bra_forward_kvds(cfg, 2, q, k, v, w, b)
    o = orc.attend_kvds(cfg, 2, q, k, v, res["idx"])
    np.testing.assert_allclose(o + orc.lepe(cfg, v, w, b), res["out"], rtol=RTOL, atol=ATOL)
    np.testing.assert_array_equal(orc.attend_kvds(cfg, 1, q, k, v, res["idx"]),
                                  orc.attend(cfg, q, k, v, res["idx"]))


def pin_kvds_window_ratio_attends_region_means(orc):
    """Ratio = window side: every routed region contributes one key and one
    value, its mean, so each query's softmax runs over the k routed region
    means of K (weights) and V (values) -- written out with numpy."""
    cfg = OracleConfig(1, 8, 8, 4, 1, 2, 3)
    rng = _rng(131)
    q, k, v = (_rand_map(rng, cfg) for _ in range(3))
    res = orc.bra_forward_kvds(cfg, 4, q, k, v)
    kb, vb = np_windows(k, 2).mean(axis=2)[0], np_windows(v, 2).mean(axis=2)[0]  # [R, C]
    qw = np_windows(q, 2)[0]  # [R, t, C]
    idx = res["idx"][0, 0]  # [R, k]
    out = np.empty_like(qw)
    for r in range(4):
        logits = qw[r] @ kb[idx[r]].T * 4 ** -0.5  # [t, k]
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[r] = (p @ vb[idx[r]]) / p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(res["out"], np_unwindows(out[None], 2, 8, 8), rtol=RTOL,
                               atol=ATOL)
    assert (res["idx"] == orc.bra_forward(cfg, q, k, v)["idx"]).all()


# ---- the projections either side of the path [P5 §五 ① and ⑧; P4 §1.1] ----
def pin_round_bf16_matches_torch(orc):
    """Rounding to bf16 agrees with torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even) on float32 inputs, ties, subnormals and
    the overflow edge."""
    rng = _rng(201)
    x = (rng.standard_normal(4096) * np.exp(rng.uniform(-30, 30, 4096))).astype(np.float32)
    specials = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130,
                         3 * 2 ** -134, 3.3895313892515355e38, 3.3961775292304e38, 0.0, -0.0,
                         1e-45], dtype=np.float32)
    x = np.concatenate([x, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_to(x.astype(np.float64), 1)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(orc.round_to(np.array([0.1, 1 / 3]), 2),
                                  np.array([0.1, 1 / 3], dtype=np.float32).astype(np.float64))


def pin_linear_matches_numpy(orc):
    """linear(x, w, b) is x w^T + b (numpy matmul, float64), for a PyTorch
    Linear weight [out, in]."""
    rng = _rng(202)
    x = rng.standard_normal((37, 48))
    w = rng.standard_normal((20, 48))
    b = rng.standard_normal(20)
    np.testing.assert_allclose(orc.linear(x, w, b), x @ w.T + b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.linear(x, w), x @ w.T, rtol=1e-12, atol=1e-12)


def pin_proj_identity_is_plain_forward(orc):
    """With w_qkv = [I; I; I], no qkv bias, w_o = I and no output bias, the
    projected forward of x is the plain forward of (x, x, x), bit for bit."""
    cfg = OracleConfig(2, 8, 8, 32, 1, 2, 2)
    rng = _rng(203)
    x = _rand_map(rng, cfg)
    w, b = _rand_lepe(rng, cfg)
    eye = np.eye(cfg.channels)
    a = orc.bra_forward_proj(cfg, 0, x, np.vstack([eye, eye, eye]), None, w, b, eye, None)
    d = orc.bra_forward(cfg, x, x, x, w, b)
    assert (a["idx"] == d["idx"]).all()
    np.testing.assert_array_equal(a["out"], d["out"])


def pin_proj_composes_linear_and_forward(orc):
    """The projected forward is linear(forward(split(round(linear(x)))))
    with every piece from numpy/torch: the qkv projection by numpy matmul and
    torch's bf16 conversion, the channel split, the plain forward, and the
    output projection by numpy matmul."""
    cfg = OracleConfig(2, 12, 8, 64, 2, 4, 3)
    rng = _rng(204)
    x = torch.from_numpy(_rand_map(rng, cfg)).to(torch.bfloat16).double().numpy()
    C = cfg.channels
    wq = rng.standard_normal((3 * C, C)) / math.sqrt(C)
    bq = rng.standard_normal(3 * C) * 0.1
    wo = rng.standard_normal((C, C)) / math.sqrt(C)
    bo = rng.standard_normal(C) * 0.1
    lw, lb = _rand_lepe(rng, cfg)
    res = orc.bra_forward_proj(cfg, 1, x, wq, bq, lw, lb, wo, bo, want_qkv=True)
    qkv = torch.from_numpy(x @ wq.T + bq).float().to(torch.bfloat16).double().numpy()
    # numpy's matmul sums in another order: a bf16 rounding may flip by one
    # step in rare halfway cases; all others agree exactly
    same = res["qkv"] == qkv
    assert same.mean() > 0.999, same.mean()
    qkv = res["qkv"]
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    plain = orc.bra_forward(cfg, q, k, v, lw, lb)
    assert (plain["idx"] == res["idx"]).all()
    np.testing.assert_allclose(res["out"], plain["out"] @ wo.T + bo, rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_topk_all_is_dense_attention,
    pin_one_region_is_dense_attention,
    pin_constant_v,
    pin_zero_k_uniform_over_lowest_regions,
    pin_means_match_numpy,
    pin_region_sums_exact_within_span,
    pin_routing_bruteforce_argsort,
    pin_ties_go_to_lower_region,
    pin_positive_scaling_keeps_routing,
    pin_routed_set_order_free,
    pin_lepe_matches_conv2d,
    pin_lepe_impulse_orientation,
    pin_hand_worked_single_token_regions,
    pin_matches_torch_recipe,
    pin_lepe_reads_v,
    pin_topk_clamp,
    pin_shared_routing_bruteforce_argsort,
    pin_shared_routing_one_head_is_per_head,
    pin_shared_routing_sums_head_affinities,
    pin_shared_ties_go_to_lower_region,
    pin_shared_matches_torch_recipe,
    pin_kv_downsample_matches_avg_pool,
    pin_kvds_ratio_one_is_plain,
    pin_kvds_all_regions_is_dense_over_pooled,
    pin_kvds_window_ratio_attends_region_means,
    pin_attend_kvds_matches_forward,
    pin_round_bf16_matches_torch,
    pin_linear_matches_numpy,
    pin_proj_identity_is_plain_forward,
    pin_proj_composes_linear_and_forward,
]
