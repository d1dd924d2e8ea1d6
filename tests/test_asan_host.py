"""The host library under AddressSanitizer (CPU only).

The library's host code (argument checking, planning, dispatch) is rebuilt
with AddressSanitizer (split_kv_attention_amd.build.build_asan: host pass
only, device code unchanged) and the host-side ABI tests run against that
build in a child process that preloads the sanitizer runtime.  Any report
(out-of-bounds access, use after free, ...) aborts the child and fails
the test.  No GPU is involved: those tests never launch a kernel.
"""
import os
import subprocess
import sys

from split_kv_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_address_sanitizer():
    lib = build.build_asan()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms, "the host code of the sanitizer build is not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["SPLITKV_LIBRARY"] = lib
    # leaks: the interpreter and the HIP runtime keep allocations until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert "AddressSanitizer" not in res.stderr + res.stdout, res.stderr[-4000:]
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout
