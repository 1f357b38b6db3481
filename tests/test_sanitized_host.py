"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The cache bookkeeping, argument checks and dispatch (host.cpp) are rebuilt by g++ with ASan
and UBSan (streaming_block_causal_amd.build.build_sanitized) and the metadata-only host tests
run against that build in a child process with the ASan runtime preloaded: every error path,
1000-chunk streams, graph bookkeeping, variable-length and editing caches.  Any sanitizer
report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_graph_host.py", "tests/test_varlen_host.py",
              "tests/test_editing_host.py", "tests/test_qkv_host.py"]


def _asan_runtime():
    if not shutil.which("g++"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_asan_runtime() is None, reason="g++ / libasan not available")
def test_host_tests_clean_under_asan_and_ubsan():
    from streaming_block_causal_amd import build
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), SWATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child checks which library it loaded, then runs the host tests
    probe = ("import streaming_block_causal_amd.native as n, sys; n.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "sys.exit(0 if n.LIB_PATH == sys.argv[1] and sys.argv[1] in maps and 'libasan' in maps else 3)")
    r = subprocess.run([sys.executable, "-c", probe, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *HOST_TESTS], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
