"""The host-side code checked under AddressSanitizer and UndefinedBehavior-
Sanitizer, CPU only: the library's C ABI entry points (host checks, workspace
sizing, layer arrays, round planning) built with both sanitizers and driven
by the host-ABI tests, and the oracle built with both and driven by its pins.
The runs go in a child process that loads clang's sanitizer runtime first;
any report fails the test."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from gated_deltanet_tree_02_amd import build as libbuild  # noqa: E402
import oracle  # noqa: E402

DRIVER = """
import sys
sys.path.insert(0, {root!r})
import gated_deltanet_tree_02_amd as gt
import oracle
gt.LIB_PATH = {lib!r}
oracle.use_library({olib!r})
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu"] + {tests!r}))
"""


def _run(tests, lib, olib):
    runtime = libbuild.asan_runtime()
    if not os.path.exists(runtime):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = DRIVER.format(root=ROOT, lib=lib, olib=olib,
                         tests=[os.path.join(ROOT, "tests", t) for t in tests])
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_host_abi_under_sanitizers():
    lib = libbuild.build_host_sanitized()
    out = _run(["test_host_abi.py"], lib, oracle.build())
    print(out.strip().splitlines()[-1])


def test_oracle_pins_under_sanitizers():
    olib = oracle.build_sanitized()
    out = _run(["test_oracle.py", "test_selective_fork_oracle.py", "test_attn_oracle.py",
                "test_fork_delta_oracle.py"], libbuild.LIB, olib)
    print(out.strip().splitlines()[-1])
