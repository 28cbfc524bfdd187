"""The C ABI from plain C: tests/c/abi_check.c is compiled against
include/*.h with the host C compiler, linked to the built library, and run
(argument validation and the host block manager; no device memory)."""

import os
import shutil
import subprocess

import pytest

from paged_kv_cache_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_compiles_links_and_passes(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = binding.lib_path()
    exe = tmp_path / "abi_check"
    build = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "abi_check.c"), lib,
                            f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", str(exe)],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
