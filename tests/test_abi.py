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
    (dict(height=256, width=256, n_win=16, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # 16 x 16 windows at C = 32: past the LDS tiles
    (dict(height=110, width=110, n_win=10, channels=64, num_heads=2),
     bra.BRA_ERR_UNSUPPORTED),                     # 11 x 11 windows at C = 64
    (dict(height=4096, width=4096, n_win=256, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # H*W = 2^24 tokens: beyond 24-bit indexing
    (dict(height=34, width=34, n_win=17, channels=32, num_heads=1),
     bra.BRA_ERR_UNSUPPORTED),                     # n_win 17: more than 256 regions
])
def test_create_rejects(lib, kw, status):
    assert bra.bra_create_status(_cfg(**kw)) == status
    assert bra.bra_last_error() != ""


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
    assert lib.bra_timing_enable(fake, 4) == bra.BRA_ERR_BAD_HANDLE
    buf = (ctypes.c_float * 2)()
    n = ctypes.c_int32()
    assert lib.bra_timing_read(fake, buf, ctypes.byref(n)) == bra.BRA_ERR_BAD_HANDLE


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(bra, "_lib", None)
    with pytest.raises(bra.BraLibraryMissing):
        bra.load_library(str(tmp_path / "libbra.so"))
