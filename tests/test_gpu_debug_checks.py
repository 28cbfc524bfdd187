"""The PA_DEBUG_CHECKS build (kernels that trap on a broken device-side
contract) gives the same results as the release build on valid inputs.  Runs
in a child process so that it loads the debug library."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_debug_check_build_matches_the_oracle(gpu_lib):
    env = dict(os.environ, PAGEDATTN_DEBUG_CHECKS="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "debug_checks_run.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
