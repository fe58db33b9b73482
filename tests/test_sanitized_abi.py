"""The host code of libbra.so under AddressSanitizer and UndefinedBehavior-
Sanitizer: the library is rebuilt with the sanitizers on its host
compilation (device code unchanged) and the ABI tests (tests/test_abi.py)
run against it in a child process that preloads the sanitizer runtime.  Any
report -- an out-of-bounds access, a use after free, undefined behaviour in
the argument checks or the handle registry -- fails the test.  No GPU is
needed: the ABI tests stop before the first kernel launch."""
import glob
import os
import subprocess
import sys

from vision_transformer_sparse_region_amd import build, build_sanitized

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = build.SOURCES + glob.glob(os.path.join(build.CSRC, "*.h")) + \
        [os.path.join(build.INCLUDE, "bra.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    lib = build_sanitized.ASAN_LIB_PATH
    if _stale(lib):
        build_sanitized.build_sanitized()
    report = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build_sanitized.asan_runtime(),
        "BRA_LIBRARY": lib,
        # the interpreter itself is not instrumented: its allocations at exit
        # would read as leaks; the handle registry's leak check is the
        # live-handle count in the allocation-failure tests
        "ASAN_OPTIONS": f"detect_leaks=0:abort_on_error=0:log_path={report}",
        "UBSAN_OPTIONS": f"print_stacktrace=1:log_path={report}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    reports = sorted(glob.glob(report + "*"))
    detail = "".join(open(p).read() for p in reports)
    assert r.returncode == 0 and not reports, r.stdout[-3000:] + r.stderr[-3000:] + detail
