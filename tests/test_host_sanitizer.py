"""The host code of the library (planning and the argument checks of every
entry point) under AddressSanitizer and UndefinedBehaviorSanitizer: a
sanitizer build of libstem (host flags only) is exercised by
_sanitized_abi.py in a child process with the ASan runtime preloaded.
CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from block_sparse_causal_amd import build as B
    lib = B.build(out=str(tmp_path / "libstem_sanitized.so"), sanitize=True)
    rt = B.sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_sanitized_abi.py"), lib, ROOT],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "sanitized ABI exercise ok" in p.stdout
