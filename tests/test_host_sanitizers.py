"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI does its argument validation, KV-metadata checks and launch plans
(split bounds, segment rule, request order, prefill tile table) on the host.
This file rebuilds the library with that host code instrumented (each
`-fsanitize=` goes to the host compilation only; the device code is the
product's), then runs the ABI test suite -- every entry point's error paths,
the host helpers against the oracle, the descriptor layout -- against it in a
child process with the sanitizer runtime preloaded.  A negative control has
the instrumented library read one element past a host array and expects the
report, so a clean run means something.  CPU only: no kernel is launched.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in the ROCm toolchain")
    from gqa_attention_sinks_amd import build
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("san")
    out = build.build(extra_flags=SAN_FLAGS, out=str(d / "libsinkattn_san.so"), build_dir=str(d / "obj"))
    return rt, out


def _run(rt, lib, args, timeout=600):
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SINKATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, *args], env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def test_abi_suite_is_clean_under_host_sanitizers(san_lib):
    rt, lib = san_lib
    r = _run(rt, lib, ["-m", "pytest", os.path.join("tests", "test_abi.py"), "-q", "-x", "-m", "not gpu",
                       "-p", "no:cacheprovider"])
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, log
    assert " passed" in r.stdout, log


NEGATIVE_CONTROL = """
import ctypes, os
import numpy as np
from gqa_attention_sinks_amd import binding
lib = binding.load_library()
assert binding.library_path() == os.environ["SINKATTN_LIB"]
kv_len = np.array([5, 70, 900], dtype=np.int32)        # three lengths ...
bounds = np.zeros((4, 2, 2), dtype=np.int32)
p = ctypes.c_void_p
lib.sinkattn_split_bounds.argtypes = [p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, p]
lib.sinkattn_split_bounds(kv_len.ctypes.data, 4, 16, 2, bounds.ctypes.data)   # ... read as four
print("not reported")
"""


def test_sanitizer_reports_a_read_past_a_host_array(san_lib):
    rt, lib = san_lib
    r = _run(rt, lib, ["-c", NEGATIVE_CONTROL], timeout=300)
    assert r.returncode != 0, r.stdout + r.stderr[-2000:]
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    assert "sinkattn_split_bounds" in r.stderr, r.stderr[-2000:]
