"""The host side of the library under AddressSanitizer (CPU only, no GPU).

Builds the library with the host code instrumented (device code is compiled as
usual) and runs the C-ABI tests against it with the sanitizer runtime
preloaded: argument validation, status strings, the allocation-failure hook and
the HIP error paths of a machine without a GPU, the slope generators, the
schedule's host side. Any invalid memory access in that host code aborts the
run. Python itself is not instrumented, so leak checking is off.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_host_code_under_address_sanitizer(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    sys.path.insert(0, ROOT)
    from alibi_linear_position_amd.build import build
    # each sanitizer flag applies to the host compilation only
    host_only = ["-Xarch_host", "-fsanitize=" + "address", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = build(out=str(tmp_path / "libalibi_host_asan.so"), extra_flags=host_only)
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms  # the host code is instrumented
    env = dict(os.environ, LD_PRELOAD=rt, ALIBI_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
