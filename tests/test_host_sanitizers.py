"""The host C++ (block allocator, prefix cache, layout) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt with instrumented host code (build.py --sanitize) and
the allocator, prefix-cache and layout parity tests of test_abi_host.py are run
against it in a child process with g++'s ASan runtime preloaded: they must pass
with no sanitizer report.  A planted overflow -- the library asked to write a
block table into a caller buffer one entry too short -- shows that the
instrumentation is live.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    try:
        path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized():
    asan = _libasan()
    if asan is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "pa_build", os.path.join(ROOT, "paged_kv_cache_424_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = mod.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=asan, PA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _child(env, args, timeout=600):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_allocator_parity_clean_under_asan_ubsan(sanitized):
    r = _child(sanitized, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py",
                           "-k", "not hip_runtime"])
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_sanitizer_catches_a_planted_overflow(sanitized):
    code = ("import numpy as np, ctypes\n"
            "import paged_kv_cache_424_amd as pa\n"
            "assert pa.LIB_PATH.endswith('sanitize/libpa.so'), pa.LIB_PATH\n"
            "a = pa.pa_allocator_create(64, 4)\n"
            "s = pa.pa_seq_create(a)\n"
            "pa.pa_seq_append_slots(a, s, 40)\n"                  # 10 blocks
            "libc = ctypes.CDLL(None)\n"
            "libc.malloc.restype = ctypes.c_void_p\n"
            "buf = ctypes.cast(libc.malloc(9 * 4), ctypes.POINTER(ctypes.c_int32))\n"   # one short; malloc: seen by ASan
            "n = ctypes.c_int32(0)\n"
            "pa._binding._lib.pa_seq_block_table(a, s, buf, 10, ctypes.byref(n))\n"
            "print('no report')\n")
    r = _child(sanitized, ["-c", code], timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode != 0 and "AddressSanitizer" in out, out[-3000:]
