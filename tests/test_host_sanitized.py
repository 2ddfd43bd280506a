"""The host code of the library (argument validation, workspace layout,
launch planning) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with the device entry points stubbed out, and
the C-ABI tests run against that build in a child process.  Any sanitizer
report aborts the child and fails this test.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_abi_suite_under_host_sanitizers(tmp_path):
    from sparse_long_document_amd import build

    lib = build.build_host_sanitized(str(tmp_path / "liblf_attn_host_asan.so"))
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["g++", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LF_ATTN_LIBRARY"] = lib
    env["LD_PRELOAD"] = " ".join(x for x in (asan, ubsan) if os.path.isabs(x))
    # Python itself is not built with the sanitizer: its allocations at exit
    # are not leaks of the library
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
