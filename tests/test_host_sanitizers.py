"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The library's host side (argument checks, tg_plan, tg_sample_budgets,
workspace sizing, launch set-up) is rebuilt with ASan and UBSan
(``build_host_sanitized``: host code only, undefined behaviour aborts), and
the host ABI tests run against it in a child process with the ASan runtime
preloaded.  Any sanitizer report fails the test.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import learned_token_pruning_score_amd._lib as L
L.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-s", "-p", "no:cacheprovider", {tests!r}])  # -s: reports reach stderr
assert L._lib is not None and L._lib._name == {lib!r}, "sanitized library was not the one loaded"
print("SANITIZED_LIBRARY_LOADED", L._lib._name)
sys.exit(rc)
"""


def _has_hipcc():
    return any(os.path.exists(p) for p in (os.environ.get("HIPCC") or "", "/opt/rocm/bin/hipcc"))


@pytest.mark.skipif(not _has_hipcc(), reason="needs hipcc to build the sanitized host library")
def test_host_abi_under_asan_and_ubsan():
    from learned_token_pruning_score_amd.build import asan_runtime, build_host_sanitized

    lib = build_host_sanitized()
    # the build really is instrumented
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = _CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_host.py"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "SANITIZED_LIBRARY_LOADED" in out
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
