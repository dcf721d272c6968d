"""The host part of the library (pack, residual quantization, LoRA extension,
unpack, size and workspace queries) under AddressSanitizer and
UndefinedBehaviorSanitizer: a g++ build of it with every finding fatal runs
the host entry points on padded and unpadded shapes in a child process with
libasan preloaded, and gives the same bytes as the regular library."""
import os
import subprocess
import sys

import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_asan_ubsan():
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan not available")
    san = B.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_asan_driver.py"), san, S.lib_path()],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "HOST_SANITIZED_OK" in r.stdout, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
