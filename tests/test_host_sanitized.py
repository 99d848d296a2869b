"""The host side of the C ABI (configuration checks, arena plan, parameter
layout, descriptor validation, error paths) under AddressSanitizer and
UBSan: the host ABI tests rerun in a child process against a build of the
library whose host code is instrumented (GPU code is not).  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

from decoder_only_gpt_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc not available")
def test_host_abi_under_asan_ubsan():
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update(GPT_TEST_LIB=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
