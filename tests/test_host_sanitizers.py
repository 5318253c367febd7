"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): argument checks and launch planning, the page table's free lists
and block-table mirror, the prefix cache's radix tree, LRU list, hash index
and arena bookkeeping.  int8_mqa_kv_amd/build_sanitized.py builds the
library with the host side instrumented; the host-library tests then run
against it in a child process that preloads the ASan runtime, and any
sanitizer report ends that process with a non-zero status."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "int8_mqa_kv_amd"))
import build_sanitized  # noqa: E402

HOST_TESTS = ["tests/test_abi.py", "tests/test_pages.py", "tests/test_prefix_cache.py"]


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(ROOT, "int8_mqa_kv_amd", "csrc", "*")) + [
        os.path.join(ROOT, "include", "mqa_kv.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already in force in this environment; not replacing it")
    try:
        runtime = build_sanitized.asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = build_sanitized.LIB
    if _stale(lib):
        build_sanitized.build()
    env = dict(os.environ, LD_PRELOAD=runtime, MQA_KV_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", *HOST_TESTS], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail, tail
    assert "runtime error:" not in tail, tail
