"""The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer
and under ThreadSanitizer, on the CPU: argument validation of every entry
point, the expert-slot pool's residency planner, and the threaded host
expert kernels of CPU-GPU co-execution with their calibration, driven by
tests/host_check.cpp (no GPU is touched).  The HIP sources are compiled with
the sanitizers on their host side only."""
import glob
import os
import subprocess

import pytest

from block_scaled_fp4_router_amd import build as ftbuild

pytestmark = pytest.mark.slow


def _runtimes_present(kind):
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.*")
    want = {"address": "libclang_rt.asan-x86_64", "thread": "libclang_rt.tsan-x86_64"}[kind]
    return any(os.path.basename(p).startswith(want) for p in libs)


@pytest.mark.parametrize("kind", ["address", "thread"])
@pytest.mark.timeout(900)
def test_host_code_under_sanitizer(kind):
    try:
        ftbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not _runtimes_present(kind):
        pytest.skip(f"no {kind} sanitizer runtime in this toolchain")
    exe = ftbuild.build_host_check(kind)
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=800)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "host checks passed" in r.stdout
