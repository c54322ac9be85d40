"""The library's host-side code under AddressSanitizer and UndefinedBehavior-
Sanitizer: a second build instruments the host code of every source
(expert_gemms_amd.build.build(sanitize=True); device code unchanged), and the
host-only CPU tests of the C ABI and the binding (argument checks, status
codes, the BLOCK_M and K-split rules, workspace sizes and layouts, the
no-allocation entry point's checks) run against it in a child process with
the ASan runtime preloaded.  Any sanitizer report fails the test: UBSan stops
at its first finding, ASan at any invalid access."""

import os
import subprocess
import sys

import pytest

from expert_gemms_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan(tmp_path):
    rt = B.asan_runtime()
    if rt is None or not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc or no ASan runtime in this toolchain")
    lib = B.build(sanitize=True)
    log = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=rt, MOE_LIBRARY=lib,
               # leaks: the interpreter's own; alloc/dealloc pairs: inside
               # uninstrumented third-party libraries
               ASAN_OPTIONS=f"detect_leaks=0:alloc_dealloc_mismatch=0:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_binding.py", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    reports = ""
    for f in os.listdir(tmp_path):
        if f.startswith("san"):
            with open(tmp_path / f) as fh:
                reports += fh.read()
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:5000])
    assert " passed" in r.stdout
