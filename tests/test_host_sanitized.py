"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``build.build_host_sanitized()`` compiles the block manager and the C API's
validation and sizing (block_manager.cpp, pa_api.cpp) with host-only ASan and
UBSan (device code as usual, no recovery from a report) and links
tests/c_abi/host_checks.cpp against them. The program drives the block
manager through seeded random operation sequences with its invariants checked
after every step, every entry point through its invalid-argument paths, and
the sizing functions at extreme sizes; it must print "ok" with no sanitizer
report. (This run found three faults, fixed with it: out-of-range pa_dtype
and pa_status values loaded as the enum type, and overflows in
pa_splitk_num_splits and pa_splitk_workspace_bytes at INT_MAX sizes.)
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_under_sanitizers():
    from paged_kv_cache_221_amd import build as pa_build
    exe = pa_build.build_host_sanitized()
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # no GPU is needed (and none is touched: every call returns before a launch)
    env["HIP_VISIBLE_DEVICES"] = ""
    p = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    report = p.stdout + p.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert p.returncode == 0 and p.stdout.strip().endswith("ok"), report[-4000:]
