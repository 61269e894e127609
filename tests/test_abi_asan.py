"""The C ABI's host code under AddressSanitizer, on the CPU: abi.cpp (the
argument checks, workspace layout and dispatch of every entry point) is
rebuilt with host ASan, and the CPU ABI tests run against that library in a
child process with the ASan runtime preloaded.  Any out-of-bounds access,
use-after-free or similar in the host code fails the run.  No GPU is used:
every call in those tests returns before launching anything."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from nvfp4_weight_only_moe_amd import binding
binding.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {testfile!r}]))
"""


def test_abi_cpu_tests_pass_under_host_asan():
    from nvfp4_weight_only_moe_amd import build_lib
    lib = build_lib.build_asan()
    # the host code really is instrumented: the library imports ASan's hooks
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm and "__asan_init" in nm
    rt = build_lib.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""            # the checks never reach a device
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                         testfile=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
