"""The C-ABI layer under host AddressSanitizer: api.cpp (argument checks, workspace layout, the
no-allocation scratch set-up) rebuilt with ASan runs the CPU ABI tests in a child process that
preloads the ASan runtime; any ASan report fails the child."""
import os
import subprocess
import sys

from mixture_experts_layer_20_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
import mixture_experts_layer_20_amd.libmoe as L
L.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_checks_clean_under_host_asan():
    lib = B.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = B.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert " passed" in r.stdout
