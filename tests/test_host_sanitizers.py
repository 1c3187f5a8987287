"""Host-side sanitizers over the C ABI's argument checks (CPU only): the
library is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code (status handling, argument validation, launch set-up; the gfx950
code objects are unchanged) and tests/test_abi.py runs against that build in
a child process with the sanitizer runtime preloaded. A report from either
sanitizer, or a failing test, fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    out = subprocess.run(["/opt/rocm/llvm/bin/clang",
                          "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_abi_checks_are_clean_under_host_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    from sparse_attention_decode_indexer_amd.build import build_host_sanitized
    lib = build_host_sanitized(str(tmp_path / "libnsa_san.so"), str(tmp_path / "obj"))
    env = dict(os.environ)
    env.update(NSA_LIB_PATH=lib, LD_PRELOAD=rt,
               # python itself is not instrumented: leak reports would be its
               # own allocations; every other finding aborts the child
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    log = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in log, log[-4000:]
    assert "runtime error:" not in log, log[-4000:]
    assert res.returncode == 0, log[-4000:]
    assert " passed" in log
