"""The C-ABI tests again with the library's host code under AddressSanitizer: argument checks,
workspace planning and error paths (everything that runs before a launch) must make no invalid
host memory access.  CPU only; builds the sanitizer build of the library when it is missing or
older than its sources."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _stale(lib, srcs):
    return not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib) for s in srcs)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitizer build")
def test_abi_tests_pass_under_host_address_sanitizer():
    from sparse_top_kv_gqa_amd import _build
    srcs = _build.sources() + [os.path.join(ROOT, "include", "spk.h")]
    if _stale(_build.LIB_ASAN, srcs):
        _build.build(asan=True)
    nm = subprocess.run(["nm", "-D", _build.LIB_ASAN], capture_output=True, text=True).stdout
    assert "__asan_report" in nm, "the sanitizer build carries no instrumentation"
    rt = _build.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, SPK_LIB=_build.LIB_ASAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
