"""ctypes binding of libbra.so (include/bra.h): the BRA forward on MI355X.

The functions carry the C names and only marshal arguments; every step of
the forward runs in the library's HIP kernels.  Torch tensors are accepted
for device memory (their data pointers are passed) and the current torch
stream is used unless a raw ``hipStream_t`` is given.

If libbra.so has not been built, loading raises ``BraLibraryMissing``: there
is no fallback path.  Build it with
``python -m vision_transformer_sparse_region_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# BRA_LIBRARY names another build of the same ABI (the host-sanitizer build
# the CPU tests use); a missing library fails loudly either way.
LIB_PATH = os.environ.get("BRA_LIBRARY", os.path.join(PKG, "libbra.so"))
HEADER = os.path.join(os.path.dirname(PKG), "include", "bra.h")

BRA_OK = 0
BRA_ERR_NULL = 1
BRA_ERR_SHAPE = 2
BRA_ERR_UNSUPPORTED = 3
BRA_ERR_HIP = 4
BRA_ERR_NOMEM = 5
BRA_ERR_BAD_HANDLE = 6
BRA_ERR_ALIGN = 7
BRA_ERR_ALIAS = 8
BRA_ERR_DEVICE = 9

BRA_F32 = 0
BRA_BF16 = 1


class BraLibraryMissing(ImportError):
    pass


class BraError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class BraConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("height", ctypes.c_int32), ("width", ctypes.c_int32),
        ("channels", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("n_win", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
        ("shared_routing", ctypes.c_int32), ("kv_downsample_ratio", ctypes.c_int32),
        ("projections", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbra.so once; raise BraLibraryMissing if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise BraLibraryMissing(
            f"{path} is not built; run `python -m vision_transformer_sparse_region_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.bra_create.argtypes = [ctypes.POINTER(BraConfig), ctypes.POINTER(vp)]
    lib.bra_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bra_forward_routed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bra_forward_proj.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bra_destroy.argtypes = [vp]
    lib.bra_topk_effective.argtypes = [vp]
    lib.bra_topk_effective.restype = i32
    lib.bra_status_string.argtypes = [ctypes.c_int]
    lib.bra_status_string.restype = ctypes.c_char_p
    lib.bra_last_error.argtypes = []
    lib.bra_last_error.restype = ctypes.c_char_p
    lib.bra_timing_enable.argtypes = [vp, i32]
    lib.bra_timing_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.bra_forward_noalloc.argtypes = [ctypes.POINTER(BraConfig), vp, vp, vp, vp, vp, vp, vp,
                                        vp]
    lib.bra_debug_inject_alloc_failure.argtypes = [i32, i32]
    lib.bra_debug_live_handles.argtypes = []
    lib.bra_debug_live_handles.restype = i32
    lib.bra_debug_projected_qkv.argtypes = [vp, vp, vp, vp, vp]
    for name in ("bra_create", "bra_forward", "bra_forward_routed", "bra_forward_proj",
                 "bra_forward_noalloc", "bra_destroy", "bra_debug_inject_alloc_failure",
                 "bra_debug_projected_qkv",
                 "bra_timing_enable", "bra_timing_read"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/bra.h declares."""
    with open(header) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(bra_\w+)\s*\(", text, re.M)))


def _check(status: int, where: str):
    if status != BRA_OK:
        lib = load_library()
        detail = lib.bra_last_error().decode() or lib.bra_status_string(status).decode()
        raise BraError(status, where, detail)


def _ptr(x):
    """Device address of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- the C functions -------------------------------------------------------

def bra_status_string(status: int) -> str:
    return load_library().bra_status_string(status).decode()


def bra_last_error() -> str:
    return load_library().bra_last_error().decode()


def bra_create(cfg: BraConfig) -> int:
    """Return a live handle (an int) or raise BraError."""
    h = ctypes.c_void_p()
    _check(load_library().bra_create(ctypes.byref(cfg), ctypes.byref(h)), "bra_create")
    return h.value


def bra_create_status(cfg) -> int:
    """Call bra_create and return the raw status (handle destroyed on success)."""
    lib = load_library()
    h = ctypes.c_void_p()
    st = lib.bra_create(ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(h))
    if st == BRA_OK:
        lib.bra_destroy(h)
    return st


def bra_forward(h: int, q, k, v, lepe_w, lepe_b, out, routing_idx=None, stream=None):
    """Enqueue the forward on the stream (torch's current stream by default)."""
    st = load_library().bra_forward(h, _ptr(q), _ptr(k), _ptr(v), _ptr(lepe_w), _ptr(lepe_b),
                                    _ptr(out), _ptr(routing_idx), _stream(stream))
    _check(st, "bra_forward")


def bra_forward_status(h, q, k, v, lepe_w, lepe_b, out, routing_idx=None, stream=0) -> int:
    """Raw status of bra_forward (for tests of the argument checks)."""
    return load_library().bra_forward(h, _ptr(q), _ptr(k), _ptr(v), _ptr(lepe_w), _ptr(lepe_b),
                                      _ptr(out), _ptr(routing_idx), stream)


def bra_forward_routed(h: int, q, k, v, lepe_w, lepe_b, routing_idx, out, stream=None):
    """Enqueue attention + LePE on a given routing (torch's current stream by default)."""
    st = load_library().bra_forward_routed(h, _ptr(q), _ptr(k), _ptr(v), _ptr(lepe_w),
                                           _ptr(lepe_b), _ptr(routing_idx), _ptr(out),
                                           _stream(stream))
    _check(st, "bra_forward_routed")


def bra_forward_routed_status(h, q, k, v, lepe_w, lepe_b, routing_idx, out, stream=0) -> int:
    """Raw status of bra_forward_routed (for tests of the argument checks)."""
    return load_library().bra_forward_routed(h, _ptr(q), _ptr(k), _ptr(v), _ptr(lepe_w),
                                             _ptr(lepe_b), _ptr(routing_idx), _ptr(out), stream)


def bra_forward_proj(h: int, x, w_qkv, b_qkv, lepe_w, lepe_b, w_o, b_o, out,
                     routing_idx=None, stream=None):
    """Enqueue the projected forward (handles created with projections)."""
    st = load_library().bra_forward_proj(h, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(lepe_w),
                                         _ptr(lepe_b), _ptr(w_o), _ptr(b_o), _ptr(out),
                                         _ptr(routing_idx), _stream(stream))
    _check(st, "bra_forward_proj")


def bra_forward_proj_status(h, x, w_qkv, b_qkv, lepe_w, lepe_b, w_o, b_o, out,
                            routing_idx=None, stream=0) -> int:
    """Raw status of bra_forward_proj (for tests of the argument checks)."""
    return load_library().bra_forward_proj(h, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(lepe_w),
                                           _ptr(lepe_b), _ptr(w_o), _ptr(b_o), _ptr(out),
                                           _ptr(routing_idx), stream)


def bra_forward_noalloc(cfg: BraConfig, q, k, v, lepe_w, lepe_b, out, routing_idx=None,
                        stream=None):
    """Enqueue the forward without a handle, on the library's device scratch array."""
    st = load_library().bra_forward_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(lepe_w), _ptr(lepe_b), _ptr(out),
                                            _ptr(routing_idx), _stream(stream))
    _check(st, "bra_forward_noalloc")


def bra_forward_noalloc_status(cfg, q, k, v, lepe_w, lepe_b, out, routing_idx=None,
                               stream=0) -> int:
    """Raw status of bra_forward_noalloc (for tests of the argument checks)."""
    return load_library().bra_forward_noalloc(ctypes.byref(cfg) if cfg is not None else None,
                                              _ptr(q), _ptr(k), _ptr(v), _ptr(lepe_w),
                                              _ptr(lepe_b), _ptr(out), _ptr(routing_idx), stream)


def bra_destroy(h) -> None:
    _check(load_library().bra_destroy(h), "bra_destroy")


def bra_topk_effective(h) -> int:
    return int(load_library().bra_topk_effective(h))


def bra_timing_enable(h, n: int) -> None:
    _check(load_library().bra_timing_enable(h, n), "bra_timing_enable")


BRA_ALLOC_HOST, BRA_ALLOC_DEVICE = 1, 2


def bra_debug_inject_alloc_failure(which: int, count: int) -> int:
    """Make the next `count` allocations of kind `which` in bra_create fail
    (a testing hook); returns the raw status."""
    return load_library().bra_debug_inject_alloc_failure(which, count)


def bra_debug_live_handles() -> int:
    return int(load_library().bra_debug_live_handles())


def bra_debug_projected_qkv_status(h, q, k, v, stream=0) -> int:
    """Raw status of bra_debug_projected_qkv (a testing hook)."""
    return load_library().bra_debug_projected_qkv(h, _ptr(q), _ptr(k), _ptr(v), stream)


KERNELS = ("region_pool", "route", "attend")


def bra_timing_read(h, capacity: int):
    """Return a list of (pool_ms, route_ms, attend_ms), one per recorded forward."""
    n = len(KERNELS)
    buf = (ctypes.c_float * (n * max(capacity, 1)))()
    cnt = ctypes.c_int32()
    _check(load_library().bra_timing_read(h, buf, ctypes.byref(cnt)), "bra_timing_read")
    return [tuple(buf[n * i + j] for j in range(n)) for i in range(cnt.value)]


# ---- convenience wrapper ---------------------------------------------------

class BRA:
    """One handle: ``BRA(batch, height, width, channels, num_heads, n_win, topk, dtype)``.

    ``forward(q, k, v, lepe_w, lepe_b)`` takes CUDA (HIP) torch tensors in NHWC,
    returns ``(out, routing_idx)``; torch only allocates the outputs.
    """

    def __init__(self, batch, height, width, channels, num_heads, n_win, topk, dtype="bf16",
                 scale=0.0, shared_routing=False, kv_downsample_ratio=1, projections=False):
        self.cfg = BraConfig(batch, height, width, channels, num_heads, n_win, topk,
                             BRA_BF16 if dtype == "bf16" else BRA_F32, scale,
                             1 if shared_routing else 0, kv_downsample_ratio,
                             1 if projections else 0)
        self.dtype = dtype
        self.route_heads = 1 if shared_routing else num_heads
        self.handle = bra_create(self.cfg)
        self.k = bra_topk_effective(self.handle)

    # The C ABI cannot see tensor sizes: every tensor handed to it is checked
    # here against the shape, dtype and device the call reads or writes.
    def _check_tensor(self, name, t, dtype, shape, device):
        if (t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or
                not t.is_cuda or t.device != device):
            raise ValueError(f"{name}: expected a contiguous {dtype} tensor {tuple(shape)} on "
                             f"{device}, got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _check_common(self, first, lepe_w, lepe_b, out, routing_idx):
        import torch
        c = self.cfg
        dev = first.device
        if lepe_w is not None:
            # lepe_w may be [C, 5, 5] or PyTorch's depthwise [C, 1, 5, 5]
            shape = (c.channels, 1, 5, 5) if lepe_w.dim() == 4 else (c.channels, 5, 5)
            self._check_tensor("lepe_w", lepe_w, torch.float32, shape, dev)
        if lepe_b is not None:
            self._check_tensor("lepe_b", lepe_b, torch.float32, (c.channels,), dev)
        if out is not None:
            self._check_tensor("out", out, first.dtype, (c.batch, c.height, c.width, c.channels),
                               dev)
        if routing_idx is not None and routing_idx is not True and routing_idx is not False:
            self._check_tensor("routing_idx", routing_idx, torch.int32,
                               (c.batch, self.route_heads, c.n_win * c.n_win, self.k), dev)

    def forward(self, q, k, v, lepe_w=None, lepe_b=None, out=None, routing_idx=True,
                stream=None):
        import torch
        c = self.cfg
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        shape = (c.batch, c.height, c.width, c.channels)
        for name, t in (("q", q), ("k", k), ("v", v)):
            self._check_tensor(name, t, want, shape, q.device)
        self._check_common(q, lepe_w, lepe_b, out, routing_idx)
        if out is None:
            out = torch.empty_like(q)
        if routing_idx is True:
            routing_idx = torch.empty((c.batch, self.route_heads, c.n_win * c.n_win, self.k),
                                      dtype=torch.int32, device=q.device)
        elif routing_idx is False:
            routing_idx = None
        bra_forward(self.handle, q, k, v, lepe_w, lepe_b, out, routing_idx, stream)
        return out, routing_idx

    def forward_routed(self, q, k, v, routing_idx, lepe_w=None, lepe_b=None, out=None,
                       stream=None):
        """Attention + LePE over the regions `routing_idx` ([B, heads, R, k] int32, or
        [B, 1, R, k] with shared routing) names."""
        import torch
        c = self.cfg
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        shape = (c.batch, c.height, c.width, c.channels)
        for name, t in (("q", q), ("k", k), ("v", v)):
            self._check_tensor(name, t, want, shape, q.device)
        if routing_idx is None or routing_idx is True or routing_idx is False:
            raise ValueError("routing_idx: a routing tensor is required")
        self._check_common(q, lepe_w, lepe_b, out, routing_idx)
        if out is None:
            out = torch.empty_like(q)
        bra_forward_routed(self.handle, q, k, v, lepe_w, lepe_b, routing_idx, out, stream)
        return out

    def forward_proj(self, x, w_qkv, w_o, b_qkv=None, b_o=None, lepe_w=None, lepe_b=None,
                     out=None, routing_idx=True, stream=None):
        """The path with the module's projections on either side (bf16; handle
        created with projections=True): returns ``(out, routing_idx)``."""
        import torch
        c = self.cfg
        shape = (c.batch, c.height, c.width, c.channels)
        self._check_tensor("x", x, torch.bfloat16, shape, x.device)
        for name, t, ws in (("w_qkv", w_qkv, (3 * c.channels, c.channels)),
                            ("w_o", w_o, (c.channels, c.channels))):
            self._check_tensor(name, t, torch.bfloat16, ws, x.device)
        for name, t, n in (("b_qkv", b_qkv, 3 * c.channels), ("b_o", b_o, c.channels)):
            if t is not None:
                self._check_tensor(name, t, torch.float32, (n,), x.device)
        self._check_common(x, lepe_w, lepe_b, out, routing_idx)
        if out is None:
            out = torch.empty_like(x)
        idx = None
        if routing_idx is True:
            idx = torch.empty((c.batch, self.route_heads, c.n_win * c.n_win, self.k),
                              dtype=torch.int32, device=x.device)
        elif routing_idx is not None and routing_idx is not False:
            idx = routing_idx
        bra_forward_proj(self.handle, x, w_qkv, b_qkv, lepe_w, lepe_b, w_o, b_o, out, idx,
                         stream)
        return out, idx

    def projected_qkv(self, stream=None):
        """The bf16 q, k, v the last forward_proj on this handle projected
        (a testing hook: copies out of the handle's workspace)."""
        import torch
        c = self.cfg
        shape = (c.batch, c.height, c.width, c.channels)
        dev = torch.device("cuda", torch.cuda.current_device())
        q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3))
        _check(bra_debug_projected_qkv_status(self.handle, q, k, v, _stream(stream)),
               "bra_debug_projected_qkv")
        return q, k, v

    def close(self):
        if self.handle:
            bra_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
