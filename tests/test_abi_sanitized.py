"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/test_abi.py (every argument check, before any HIP call) runs in a child
process against libfa_hostsan.so -- the same sources with the host code
instrumented and the device code unchanged -- with the sanitizer runtime
preloaded. A memory error or undefined behaviour in the validation aborts
the child, which fails this test."""

import os
import subprocess
import sys

from tests.gpu_util import ROOT
from exact_attention_109_amd import _build


def test_abi_under_host_sanitizers():
    lib = _build.VARIANTS["hostsan"][0]
    if not os.path.exists(lib):
        _build.build(variant="hostsan")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "library is not instrumented"
    rt = _build.sanitizer_runtime()
    assert os.path.isfile(rt), rt
    env = dict(os.environ, FA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
