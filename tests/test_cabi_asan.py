"""The C-ABI checks of tests/test_cabi.py against an AddressSanitizer build of
the library's host code (CPU only; no GPU code is instrumented).

Every argument check, descriptor read, size computation and error path of the
entry points runs in host code before any launch; this test builds libpa.so
again with ASan on the host side only (each sanitizer flag after -Xarch_host),
preloads the clang ASan runtime into a fresh interpreter, points the binding
at that build (PA_LIB_PATH) and runs tests/test_cabi.py there.  Any invalid
host memory access aborts that run with an ASan report.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
HOST_ASAN_LINK = "-Xarch_host -fsanitize=address -Xarch_host -shared-libasan".split()


def _runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rt[-1] if rt else None


@pytest.mark.timeout(900)
def test_cabi_checks_under_host_asan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    sys.path.insert(0, ROOT)
    from decode_attention_paged_pa_amd.build import build

    lib = str(tmp_path / "libpa_asan.so")
    build(extra_flags=HOST_ASAN, link_flags=HOST_ASAN_LINK, out_path=lib)
    env = dict(os.environ, LD_PRELOAD=rt, PA_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    # the runtime is live in that interpreter, and the build is instrumented
    probe = subprocess.run(
        [sys.executable, "-c", "import ctypes; ctypes.CDLL(None).__asan_report_load1; "
                               "assert hasattr(ctypes.CDLL(%r), '__asan_init')" % lib],
        env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_cabi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout
