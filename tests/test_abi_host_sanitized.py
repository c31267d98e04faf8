"""The C-ABI's host code (argument validation, planning, workspace layout)
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

libflce_hostsan.so is the library built with the host side instrumented
(`python -m linear_cross_entropy_tiled_amd.build --host-sanitizers`); the
host-side ABI and binding tests run against it in a child process with the
shared ASan runtime preloaded, and any report aborts that process.  (The idea
of checking every argument before a launch follows quack-kernels'
chunked_linear_cross_entropy, which validates its inputs up front.)"""
import os
import subprocess
import sys

import pytest

from linear_cross_entropy_tiled_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    try:
        build.hipcc()
        rt = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)] + [os.path.join(ROOT, "include", "flce.h")]
    newest = max(os.path.getmtime(f) for f in srcs)
    if not os.path.exists(build.SAN_LIB_PATH) or os.path.getmtime(build.SAN_LIB_PATH) < newest:
        build.build_host_sanitized()
    env = dict(os.environ)
    env.update(FLCE_LIB_PATH=build.SAN_LIB_PATH, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_the_sanitized_library_is_instrumented_and_loaded(san_env):
    nm = subprocess.run(["nm", "-D", "--undefined-only", build.SAN_LIB_PATH], stdout=subprocess.PIPE, check=True)
    syms = nm.stdout.decode()
    assert "__asan_report_" in syms and "__ubsan_handle_" in syms
    code = ("import linear_cross_entropy_tiled_amd as f; f.load(); "
            "m = open('/proc/self/maps').read(); "
            "print('hostsan' if 'libflce_hostsan.so' in m and 'libclang_rt.asan' in m else 'missing')")
    r = subprocess.run([sys.executable, "-c", code], env=san_env, cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, timeout=600)
    assert r.stdout.decode().strip().endswith("hostsan"), r.stdout.decode()[-2000:]


def test_host_abi_tests_pass_under_asan_and_ubsan(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "tests/test_binding_validation.py"],
                       env=san_env, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=900)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
