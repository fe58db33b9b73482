"""CPU oracle of the Bi-Level Routing Attention forward pass (fp64, plain C).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
package never does, and shares no code with it.

This module is the ctypes front of ``liboracle.so`` (built from
``bra_oracle.c`` by ``oracle.build.build_oracle``).  Every array argument is
converted to a C-contiguous float64 (or int32) numpy copy; the functions
return new numpy arrays.  Layouts are those of ``bra_oracle.h``:
q/k/v/out ``[B, H, W, C]``, means ``[B, heads, R, head_dim]``, affinity
``[B, heads, R, R]``, routing ``[B, heads, R, k]`` (int32), LePE weight
``[C, 5, 5]`` and bias ``[C]``.

``OracleLib(path)`` wraps one build of the library (the tests also load
deliberately broken builds through it, to show that the pins catch them); the
module-level functions use the default build.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from .build import LIB_PATH, build_oracle

__all__ = [
    "OracleConfig", "OracleLib", "topk_effective", "region_means", "route", "attend", "lepe",
    "attend_with_routing", "bra_forward", "num_threads", "default", "round_to", "linear",
    "bra_forward_proj",
]


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("height", ctypes.c_int32), ("width", ctypes.c_int32),
        ("channels", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("n_win", ctypes.c_int32), ("topk", ctypes.c_int32), ("scale", ctypes.c_double),
    ]


@dataclass(frozen=True)
class OracleConfig:
    batch: int
    height: int
    width: int
    channels: int
    num_heads: int
    n_win: int
    topk: int
    scale: float = 0.0  # <= 0: head_dim ** -0.5

    @property
    def head_dim(self) -> int:
        return self.channels // self.num_heads

    @property
    def regions(self) -> int:
        return self.n_win * self.n_win

    def _c(self) -> _Cfg:
        return _Cfg(self.batch, self.height, self.width, self.channels, self.num_heads,
                    self.n_win, self.topk, float(self.scale))


_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)


def _f64(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return arr, arr.ctypes.data_as(_DP)


def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_IP)


def _ptr(a):
    return a.ctypes.data_as(_DP) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected the configuration")


def _map_shape(cfg: OracleConfig):
    return (cfg.batch, cfg.height, cfg.width, cfg.channels)


def _bar_shape(cfg: OracleConfig):
    return (cfg.batch, cfg.num_heads, cfg.regions, cfg.head_dim)


class OracleLib:
    """One loaded build of liboracle.so."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        cp = ctypes.POINTER(_Cfg)
        lib.oracle_topk_effective.argtypes = [cp]
        lib.oracle_topk_effective.restype = ctypes.c_int32
        lib.oracle_region_means.argtypes = [cp, _DP, _DP]
        lib.oracle_route.argtypes = [cp, _DP, _DP, _DP, _IP]
        lib.oracle_attend.argtypes = [cp, _DP, _DP, _DP, _IP, _DP]
        lib.oracle_lepe.argtypes = [cp, _DP, _DP, _DP, _DP]
        lib.oracle_attend_with_routing.argtypes = [cp, _DP, _DP, _DP, _DP, _DP, _IP, _DP]
        lib.oracle_bra_forward.argtypes = [cp, _DP, _DP, _DP, _DP, _DP, _DP, _IP, _DP, _DP,
                                           _DP]
        lib.oracle_route_shared.argtypes = [cp, _DP, _DP, _DP, _IP]
        lib.oracle_bra_forward_shared.argtypes = [cp, _DP, _DP, _DP, _DP, _DP, _DP, _IP, _DP]
        lib.oracle_kv_downsample.argtypes = [cp, ctypes.c_int, _DP, _DP]
        lib.oracle_bra_forward_kvds.argtypes = [cp, ctypes.c_int, _DP, _DP, _DP, _DP, _DP, _DP,
                                                _IP]
        lib.oracle_attend_kvds.argtypes = [cp, ctypes.c_int, _DP, _DP, _DP, _IP, _DP]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_round.argtypes = [ctypes.c_int, ctypes.c_int64, _DP, _DP]
        lib.oracle_linear.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, _DP, _DP, _DP,
                                      ctypes.c_int, _DP]
        lib.oracle_bra_forward_proj.argtypes = [cp, ctypes.c_int, _DP, _DP, _DP, _DP, _DP, _DP,
                                                _DP, _DP, _IP, _DP]
        for name in ("oracle_region_means", "oracle_route", "oracle_attend", "oracle_lepe",
                     "oracle_attend_with_routing", "oracle_bra_forward", "oracle_route_shared",
                     "oracle_bra_forward_shared", "oracle_kv_downsample",
                     "oracle_bra_forward_kvds", "oracle_attend_kvds", "oracle_num_threads",
                     "oracle_round", "oracle_linear", "oracle_bra_forward_proj"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def topk_effective(self, cfg: OracleConfig) -> int:
        c = cfg._c()
        return int(self.lib.oracle_topk_effective(ctypes.byref(c)))

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def region_means(self, cfg: OracleConfig, x) -> np.ndarray:
        c = cfg._c()
        xa, xp = _f64(x)
        out = np.empty(_bar_shape(cfg), np.float64)
        _check(self.lib.oracle_region_means(ctypes.byref(c), xp, _ptr(out)), "region_means")
        return out

    def route(self, cfg: OracleConfig, qbar, kbar, want_aff: bool = False):
        """Return idx [B,h,R,k] (and the affinity [B,h,R,R] if want_aff)."""
        c = cfg._c()
        qa, qp = _f64(qbar)
        ka, kp = _f64(kbar)
        k = self.topk_effective(cfg)
        idx = np.empty((cfg.batch, cfg.num_heads, cfg.regions, k), np.int32)
        aff = np.empty((cfg.batch, cfg.num_heads, cfg.regions, cfg.regions), np.float64) \
            if want_aff else None
        _check(self.lib.oracle_route(ctypes.byref(c), qp, kp, _ptr(aff),
                                     idx.ctypes.data_as(_IP)), "route")
        return (idx, aff) if want_aff else idx

    def route_shared(self, cfg: OracleConfig, qbar, kbar, want_aff: bool = False):
        """Head-shared routing: idx [B,R,k] (and the affinity [B,R,R] if want_aff)."""
        c = cfg._c()
        qa, qp = _f64(qbar)
        ka, kp = _f64(kbar)
        k = self.topk_effective(cfg)
        idx = np.empty((cfg.batch, cfg.regions, k), np.int32)
        aff = np.empty((cfg.batch, cfg.regions, cfg.regions), np.float64) if want_aff else None
        _check(self.lib.oracle_route_shared(ctypes.byref(c), qp, kp, _ptr(aff),
                                            idx.ctypes.data_as(_IP)), "route_shared")
        return (idx, aff) if want_aff else idx

    def bra_forward_shared(self, cfg: OracleConfig, q, k, v, w=None, b=None, *,
                           want_aff=False):
        """Whole forward with head-shared routing: dict with 'out', 'idx' [B,R,k]
        (+ 'aff' [B,R,R])."""
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        kk = self.topk_effective(cfg)
        out = np.empty(_map_shape(cfg), np.float64)
        idx = np.empty((cfg.batch, cfg.regions, kk), np.int32)
        aff = np.empty((cfg.batch, cfg.regions, cfg.regions), np.float64) if want_aff else None
        _check(self.lib.oracle_bra_forward_shared(ctypes.byref(c), qp, kp, vp, wp, bp,
                                                  _ptr(out), idx.ctypes.data_as(_IP),
                                                  _ptr(aff)), "bra_forward_shared")
        res = {"out": out, "idx": idx}
        if want_aff:
            res["aff"] = aff
        return res

    def kv_downsample(self, cfg: OracleConfig, ratio: int, x) -> np.ndarray:
        c = cfg._c()
        xa, xp = _f64(x)
        out = np.empty((cfg.batch, cfg.height // ratio, cfg.width // ratio, cfg.channels),
                       np.float64)
        _check(self.lib.oracle_kv_downsample(ctypes.byref(c), ratio, xp, _ptr(out)),
               "kv_downsample")
        return out

    def attend_kvds(self, cfg: OracleConfig, ratio: int, q, k, v, idx) -> np.ndarray:
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        ia, ip = _i32(idx)
        out = np.empty(_map_shape(cfg), np.float64)
        _check(self.lib.oracle_attend_kvds(ctypes.byref(c), ratio, qp, kp, vp, ip, _ptr(out)),
               "attend_kvds")
        return out

    def bra_forward_kvds(self, cfg: OracleConfig, ratio: int, q, k, v, w=None, b=None):
        """Whole forward with KV downsampling: dict with 'out' and 'idx'."""
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        kk = self.topk_effective(cfg)
        out = np.empty(_map_shape(cfg), np.float64)
        idx = np.empty((cfg.batch, cfg.num_heads, cfg.regions, kk), np.int32)
        _check(self.lib.oracle_bra_forward_kvds(ctypes.byref(c), ratio, qp, kp, vp, wp, bp,
                                                _ptr(out), idx.ctypes.data_as(_IP)),
               "bra_forward_kvds")
        return {"out": out, "idx": idx}

    def attend(self, cfg: OracleConfig, q, k, v, idx) -> np.ndarray:
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        ia, ip = _i32(idx)
        out = np.empty(_map_shape(cfg), np.float64)
        _check(self.lib.oracle_attend(ctypes.byref(c), qp, kp, vp, ip, _ptr(out)), "attend")
        return out

    def lepe(self, cfg: OracleConfig, v, w, b=None) -> np.ndarray:
        c = cfg._c()
        va, vp = _f64(v)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        out = np.empty(_map_shape(cfg), np.float64)
        _check(self.lib.oracle_lepe(ctypes.byref(c), vp, wp, bp, _ptr(out)), "lepe")
        return out

    def attend_with_routing(self, cfg: OracleConfig, q, k, v, w, b, idx) -> np.ndarray:
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        ia, ip = _i32(idx)
        out = np.empty(_map_shape(cfg), np.float64)
        _check(self.lib.oracle_attend_with_routing(ctypes.byref(c), qp, kp, vp, wp, bp, ip,
                                                   _ptr(out)), "attend_with_routing")
        return out

    def bra_forward(self, cfg: OracleConfig, q, k, v, w=None, b=None, *, want_aff=False,
                    want_means=False):
        """Whole forward; returns a dict with 'out', 'idx' (+ 'aff', 'qbar', 'kbar')."""
        c = cfg._c()
        qa, qp = _f64(q)
        ka, kp = _f64(k)
        va, vp = _f64(v)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        kk = self.topk_effective(cfg)
        out = np.empty(_map_shape(cfg), np.float64)
        idx = np.empty((cfg.batch, cfg.num_heads, cfg.regions, kk), np.int32)
        aff = np.empty((cfg.batch, cfg.num_heads, cfg.regions, cfg.regions), np.float64) \
            if want_aff else None
        qbar = np.empty(_bar_shape(cfg), np.float64) if want_means else None
        kbar = np.empty(_bar_shape(cfg), np.float64) if want_means else None
        _check(self.lib.oracle_bra_forward(ctypes.byref(c), qp, kp, vp, wp, bp, _ptr(out),
                                           idx.ctypes.data_as(_IP), _ptr(aff), _ptr(qbar),
                                           _ptr(kbar)), "bra_forward")
        res = {"out": out, "idx": idx}
        if want_aff:
            res["aff"] = aff
        if want_means:
            res["qbar"], res["kbar"] = qbar, kbar
        return res


    # ---- projections (round: 0 none, 1 bf16, 2 fp32) -----------------------
    ROUND = {"f64": 0, "bf16": 1, "f32": 2}

    def round_to(self, x, round_mode: int):
        xa, xp = _f64(x)
        y = np.empty_like(xa)
        _check(self.lib.oracle_round(int(round_mode), xa.size, xp, _ptr(y)), "round")
        return y

    def linear(self, x, w, b=None, round_mode: int = 0):
        """y[..., o] = x[..., :] . w[o, :] + b[o] (w a Linear weight [out, in])."""
        xa, xp = _f64(x)
        wa, wp = _f64(w)
        ba, bp = _f64(b)
        out_f, in_f = wa.shape
        rows = xa.size // in_f
        y = np.empty(xa.shape[:-1] + (out_f,), np.float64)
        _check(self.lib.oracle_linear(rows, in_f, out_f, xp, wp, bp, int(round_mode), _ptr(y)),
               "linear")
        return y

    def bra_forward_proj(self, cfg: OracleConfig, round_mode: int, x, w_qkv, b_qkv, lepe_w,
                         lepe_b, w_o, b_o, *, want_qkv=False):
        """Projections + forward; returns a dict with 'out', 'idx' (+ 'qkv')."""
        c = cfg._c()
        arrs = [_f64(a) for a in (x, w_qkv, b_qkv, lepe_w, lepe_b, w_o, b_o)]
        kk = self.topk_effective(cfg)
        out = np.empty(_map_shape(cfg), np.float64)
        idx = np.empty((cfg.batch, cfg.num_heads, cfg.regions, kk), np.int32)
        qkv = np.empty(_map_shape(cfg)[:-1] + (3 * cfg.channels,), np.float64) \
            if want_qkv else None
        _check(self.lib.oracle_bra_forward_proj(ctypes.byref(c), int(round_mode),
                                                *[p for _, p in arrs], _ptr(out),
                                                idx.ctypes.data_as(_IP), _ptr(qkv)),
               "bra_forward_proj")
        res = {"out": out, "idx": idx}
        if want_qkv:
            res["qkv"] = qkv
        return res


_default = None


def default() -> OracleLib:
    """The default build, compiled first only if it is not there yet."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build_oracle()
        _default = OracleLib(LIB_PATH)
    return _default


def topk_effective(cfg):
    return default().topk_effective(cfg)


def num_threads():
    return default().num_threads()


def region_means(cfg, x):
    return default().region_means(cfg, x)


def route(cfg, qbar, kbar, want_aff=False):
    return default().route(cfg, qbar, kbar, want_aff)


def attend(cfg, q, k, v, idx):
    return default().attend(cfg, q, k, v, idx)


def lepe(cfg, v, w, b=None):
    return default().lepe(cfg, v, w, b)


def attend_with_routing(cfg, q, k, v, w, b, idx):
    return default().attend_with_routing(cfg, q, k, v, w, b, idx)


def bra_forward(cfg, q, k, v, w=None, b=None, *, want_aff=False, want_means=False):
    return default().bra_forward(cfg, q, k, v, w, b, want_aff=want_aff, want_means=want_means)


def route_shared(cfg, qbar, kbar, want_aff=False):
    return default().route_shared(cfg, qbar, kbar, want_aff)


def bra_forward_shared(cfg, q, k, v, w=None, b=None, *, want_aff=False):
    return default().bra_forward_shared(cfg, q, k, v, w, b, want_aff=want_aff)


def kv_downsample(cfg, ratio, x):
    return default().kv_downsample(cfg, ratio, x)


def bra_forward_kvds(cfg, ratio, q, k, v, w=None, b=None):
    return default().bra_forward_kvds(cfg, ratio, q, k, v, w, b)


def attend_kvds(cfg, ratio, q, k, v, idx):
    return default().attend_kvds(cfg, ratio, q, k, v, idx)


def round_to(x, round_mode):
    return default().round_to(x, round_mode)


def linear(x, w, b=None, round_mode=0):
    return default().linear(x, w, b, round_mode)


def bra_forward_proj(cfg, round_mode, x, w_qkv, b_qkv, lepe_w, lepe_b, w_o, b_o, *,
                     want_qkv=False):
    return default().bra_forward_proj(cfg, round_mode, x, w_qkv, b_qkv, lepe_w, lepe_b, w_o,
                                      b_o, want_qkv=want_qkv)
