"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: every argument-check and planning case of
test_abi.py runs against a build whose host code (api, mla, append) carries
both sanitizers, in a child process with the sanitizer runtime preloaded.
Any report (a read or write out of bounds, an overflow, a bad shift) ends
that process with an error.  No GPU is needed: the cases never launch."""

import os
import shutil
import subprocess
import sys

import pytest

from decode_attention_kv_attn_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(build.HIPCC) or build.sanitizer_runtime() is None,
                    reason="hipcc or the clang sanitizer runtime is missing")
def test_abi_cases_under_host_sanitizers():
    lib = build.build_host_sanitized()
    assert "__asan_report" in subprocess.run(
        ["nm", "-D", lib], capture_output=True, text=True).stdout
    env = build.host_sanitizer_env()
    code = ("import ctypes, sys; ctypes.CDLL(None).__asan_init; "
            "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
            "'tests/test_abi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
