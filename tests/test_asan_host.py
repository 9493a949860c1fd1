"""The C ABI's host code under AddressSanitizer (CPU only).

The library is rebuilt with the host side of every compile instrumented (device code unchanged),
and the CPU boundary suite runs against it in a child process that preloads the sanitizer runtime:
handle creation and destruction, the size and workspace queries, the plan override, every host
error path of the entry points, status strings and error details.  Any heap, stack or global
out-of-bounds access, use after free or double free in that code fails the test.  (Two boundary
tests are left out: one caps the address space, which the sanitizer's shadow memory cannot live
under, and one runs bench.py, which needs no library.)
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_boundary_suite_under_address_sanitizer(tmp_path):
    from int8_kv_cache_hkv_amd import build as B
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    pkg = tmp_path / "int8_kv_cache_hkv_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(B.PKG, "__init__.py"), pkg)
    lib = B.build(out=str(pkg / "libhkv.so"), host_flags=("-fsanitize=address", "-fno-omit-frame-pointer"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:exitcode=99",
               PYTHONPATH=f"{tmp_path}{os.pathsep}{B.ROOT}")
    probe = subprocess.run([sys.executable, "-c", "import int8_kv_cache_hkv_amd as h; print(h.LIB_PATH)"],
                           env=env, cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-3000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "--import-mode=append",
                          "-m", "not gpu", os.path.join(B.ROOT, "tests", "test_boundary.py"),
                          "-k", "not allocation_failure and not bench_refuses"],
                         env=env, cwd=tmp_path, capture_output=True, text=True, timeout=600)
    text = res.stdout + res.stderr
    assert res.returncode == 0 and "AddressSanitizer" not in text, text[-5000:]
    assert " passed" in res.stdout
