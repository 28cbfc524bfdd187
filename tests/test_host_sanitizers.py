"""Host code under AddressSanitizer and UBSan (CPU only, no GPU work).

* The block manager (csrc/block_manager.cpp) with a random new / fork /
  append / free fuzz on pools of one-block and multi-block pages: every live
  sequence must read back its own token history after every step, through a
  simulated pool that receives the copy-on-write copies and the appends
  (tests/c/bm_fuzz.cpp).
* The C ABI's host-side argument checking (csrc/api.hip, kernel launchers
  stubbed out) under random argument vectors through every entry point
  (tests/c/abi_fuzz.cpp).

Sanitizers apply to host code only: on each hipcc line every -fsanitize= goes
behind -Xarch_host, so no device code is built with them.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_attn_amd", "csrc")
CDIR = os.path.join(ROOT, "tests", "c")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _build(tmp_path, name, sources, device=False):
    cmd = [_hipcc(), "-O1", "-g", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}", *SAN]
    if device:
        cmd += ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    exe = str(tmp_path / name)
    r = subprocess.run(cmd + sources + ["-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r.stdout


def test_block_manager_fuzz_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "bm_fuzz", [os.path.join(CDIR, "bm_fuzz.cpp"), os.path.join(CSRC, "block_manager.cpp")])
    out = _run(exe, 200, 300)
    assert "block manager fuzz: 200 pools" in out


def test_abi_argument_checks_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "abi_fuzz", [os.path.join(CSRC, "api.hip"), os.path.join(CDIR, "launch_stubs.cpp"),
                                        os.path.join(CDIR, "abi_fuzz.cpp")], device=True)
    env_free = _run(exe, 200000)
    assert "200000 calls" in env_free
