"""Host-side checks of the C ABI (no kernel runs): the library loads, exports
every function include/bra.h declares, and rejects bad arguments with the
documented status codes before touching the GPU."""
import ctypes

import pytest

from vision_transformer_sparse_region_amd import bra


@pytest.fixture(scope="module")
def lib():
    return bra.load_library()


def test_exports_every_declared_function(lib):
    names = bra.declared_functions()
    assert {"bra_create", "bra_forward", "bra_destroy"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(10):
        s = bra.bra_status_string(code)
        assert s and s != "unknown status"
    assert bra.bra_status_string(99) == "unknown status"


def _cfg(**kw):
    base = dict(batch=2, height=28, width=28, channels=64, num_heads=2, n_win=7, topk=4,
                dtype=bra.BRA_BF16, scale=0.0)
    base.update(kw)
    return bra.BraConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), bra.BRA_ERR_SHAPE),
    (dict(height=-4), bra.BRA_ERR_SHAPE),
    (dict(n_win=0), bra.BRA_ERR_SHAPE),
    (dict(height=30), bra.BRA_ERR_SHAPE),          # 30 % 7 != 0
    (dict(width=27), bra.BRA_ERR_SHAPE),
    (dict(channels=65), bra.BRA_ERR_SHAPE),        # not divisible by heads
    (dict(channels=64, num_heads=4), bra.BRA_ERR_UNSUPPORTED),   # head_dim 16
    (dict(channels=128, num_heads=2), bra.BRA_ERR_UNSUPPORTED),  # head_dim 64
    (dict(dtype=7), bra.BRA_ERR_UNSUPPORTED),
    (dict(height=256, width=256, n_win=1, channels=32, num_heads=1, topk=1),
     bra.BRA_ERR_UNSUPPORTED),                     # one 65536-token region does not fit on chip
    (dict(height=65536, width=65536, n_win=1, channels=32, num_heads=1), bra.BRA_ERR_SHAPE),
    (dict(shared_routing=2), bra.BRA_ERR_SHAPE),   # a flag: 0 or 1
    (dict(projections=2), bra.BRA_ERR_SHAPE),      # a flag: 0 or 1
    (dict(projections=1, dtype=bra.BRA_F32), bra.BRA_ERR_UNSUPPORTED),  # bf16 only
    (dict(projections=1, shared_routing=1), bra.BRA_ERR_UNSUPPORTED),  # per-head routing only
    (dict(projections=1, kv_downsample_ratio=2), bra.BRA_ERR_UNSUPPORTED),  # no KV downsampling
    (dict(projections=1, channels=544, num_heads=17), bra.BRA_ERR_UNSUPPORTED),  # C <= 512
    (dict(kv_downsample_ratio=3), bra.BRA_ERR_SHAPE),  # 3 does not divide the 4x4 windows
    (dict(height=108, width=108, n_win=4, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # 27 x 27 windows at C = 32: past 160 KB of LDS
    (dict(height=76, width=76, n_win=4, channels=64, num_heads=2),
     bra.BRA_ERR_UNSUPPORTED),                     # 19 x 19 windows at C = 64
    (dict(height=72, width=72, n_win=8, channels=256, num_heads=8),
     bra.BRA_ERR_UNSUPPORTED),                     # 9 x 9 windows at C = 256
    (dict(height=60, width=60, n_win=4, channels=128, num_heads=4, dtype=bra.BRA_F32),
     bra.BRA_ERR_UNSUPPORTED),                     # fp32: 15 x 15 windows at C = 128
    (dict(height=4096, width=4096, n_win=256, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # H*W = 2^24 tokens: beyond 24-bit indexing
    (dict(height=34, width=34, n_win=17, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # n_win 17: more than 256 regions
])
def test_create_rejects(lib, kw, status):
    assert bra.bra_create_status(_cfg(**kw)) == status
    assert bra.bra_last_error() != ""


@pytest.mark.parametrize("kw", [
    # "从静态到动态" §4.1: dim 128, n_win 7, topk 4, kv_downsample_ratio 4, on a
    # 56 x 56 map with 4 heads of 32
    dict(channels=128, num_heads=4, height=56, width=56, topk=4, kv_downsample_ratio=4),
    # the segmentation module of "【医学图像分割模块】BiFormer" §六: dim 256, 8 heads,
    # n_win 7, topk 4 (on a 56 x 56 map; the page gives none)
    dict(channels=256, num_heads=8, height=56, width=56, topk=4),
    dict(height=64, width=64, n_win=4, channels=64, num_heads=2),    # 16 x 16 windows
    dict(height=104, width=104, n_win=4, channels=32, num_heads=1),  # 26 x 26 windows
    dict(height=72, width=72, n_win=4, channels=64, num_heads=2),    # 18 x 18 windows
    dict(height=48, width=48, n_win=8, channels=256, num_heads=8, dtype=bra.BRA_F32),
], ids=["page_dim128_kvds4", "page_dim256_heads8", "win16_c64", "win26_c32", "win18_c64",
        "f32_window6_c256"])
def test_create_accepts_tiles_up_to_160_kb(lib, kw):
    """Tiles above 64 KB and up to the CU's 160 KB of LDS pass the checks
    (without a GPU, creation then stops at the first HIP call)."""
    st = bra.bra_create_status(_cfg(**kw))
    assert st not in (bra.BRA_ERR_UNSUPPORTED, bra.BRA_ERR_SHAPE), bra.bra_last_error()


def test_create_null_arguments(lib):
    assert lib.bra_create(None, ctypes.byref(ctypes.c_void_p())) == bra.BRA_ERR_NULL
    c = _cfg()
    assert lib.bra_create(ctypes.byref(c), None) == bra.BRA_ERR_NULL


def test_dead_handles(lib):
    fake = 0x1234560
    assert lib.bra_destroy(None) == bra.BRA_OK
    assert lib.bra_destroy(fake) == bra.BRA_ERR_BAD_HANDLE
    assert bra.bra_forward_status(fake, 16, 16, 16, None, None, 32) == bra.BRA_ERR_BAD_HANDLE
    assert bra.bra_forward_routed_status(fake, 16, 16, 16, None, None, 16, 32) == \
        bra.BRA_ERR_BAD_HANDLE
    assert bra.bra_forward_proj_status(fake, 16, 16, None, None, None, 16, None, 32) == \
        bra.BRA_ERR_BAD_HANDLE
    assert lib.bra_topk_effective(fake) == -1
    assert bra.bra_debug_projected_qkv_status(fake, 16, 16, 16) == bra.BRA_ERR_BAD_HANDLE
    assert lib.bra_timing_enable(fake, 4) == bra.BRA_ERR_BAD_HANDLE
    buf = (ctypes.c_float * 2)()
    n = ctypes.c_int32()
    assert lib.bra_timing_read(fake, buf, ctypes.byref(n)) == bra.BRA_ERR_BAD_HANDLE


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(bra, "_lib", None)
    with pytest.raises(bra.BraLibraryMissing):
        bra.load_library(str(tmp_path / "libbra.so"))


@pytest.mark.parametrize("which", [bra.BRA_ALLOC_HOST, bra.BRA_ALLOC_DEVICE],
                         ids=["handle", "workspace"])
def test_create_reports_allocation_failure_and_leaks_nothing(lib, which):
    """An injected allocation failure makes bra_create return BRA_ERR_NOMEM,
    leave *out NULL and keep no handle alive; the hook disarms after its
    count.  (The failure is injected before any HIP call, so this runs
    without a GPU; the host-sanitizer build of the library runs it too.)"""
    live = bra.bra_debug_live_handles()
    assert bra.bra_debug_inject_alloc_failure(which, 2) == bra.BRA_OK
    for _ in range(2):
        h = ctypes.c_void_p(0x1)
        c = _cfg()
        assert lib.bra_create(ctypes.byref(c), ctypes.byref(h)) == bra.BRA_ERR_NOMEM
        assert h.value is None
        assert "out of memory" in bra.bra_last_error() or "host allocation" in bra.bra_last_error()
        assert bra.bra_debug_live_handles() == live
    # disarmed: the next create gets past the allocation (on a CPU host it
    # then fails at the first HIP call, never with BRA_ERR_NOMEM)
    st = bra.bra_create_status(_cfg())
    assert st != bra.BRA_ERR_NOMEM
    assert bra.bra_debug_live_handles() == live


def test_alloc_failure_hook_arguments(lib):
    assert bra.bra_debug_inject_alloc_failure(bra.BRA_ALLOC_HOST, -1) == bra.BRA_ERR_SHAPE
    assert bra.bra_debug_inject_alloc_failure(7, 1) == bra.BRA_ERR_SHAPE
    assert bra.bra_debug_inject_alloc_failure(bra.BRA_ALLOC_DEVICE, 0) == bra.BRA_OK


def test_noalloc_rejects_before_touching_the_gpu(lib):
    """bra_forward_noalloc checks its config and pointers, and the workspace
    size against its fixed scratch array, before any HIP call."""
    assert bra.bra_forward_noalloc_status(None, 16, 16, 16, None, None, 32) == bra.BRA_ERR_NULL
    assert bra.bra_forward_noalloc_status(_cfg(batch=0), 16, 16, 16, None, None, 32) == \
        bra.BRA_ERR_SHAPE
    assert bra.bra_forward_noalloc_status(_cfg(projections=1), 16, 16, 16, None, None, 32) == \
        bra.BRA_ERR_UNSUPPORTED
    assert bra.bra_forward_noalloc_status(_cfg(), 16, 16, 16, None, None, 16) == \
        bra.BRA_ERR_ALIAS
    # 512 images of 56 x 56 with per-head routing: 16 MB of region means alone
    big = _cfg(batch=512, height=56, width=56, channels=64, num_heads=2, n_win=7, topk=1)
    assert bra.bra_forward_noalloc_status(big, 16, 1 << 40, 2 << 40, None, None, 3 << 40) == \
        bra.BRA_ERR_UNSUPPORTED
    assert "scratch" in bra.bra_last_error()
