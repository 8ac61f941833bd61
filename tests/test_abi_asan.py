"""The host-side tests of the C ABI (argument validation, workspace sizing,
plan errors) run again against a build of libvla whose host runtime is
compiled with AddressSanitizer; any ASan report fails the run. CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_host_tests_are_clean_under_asan():
    ba = pytest.importorskip("vla_robot_policy_amd.build_asan")
    try:
        ba.build_asan()
    except (RuntimeError, FileNotFoundError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no ASan toolchain here: {e}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=ba.asan_env(), capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
