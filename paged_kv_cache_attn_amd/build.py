"""Build the gfx950 shared library ``libpagedattn.so`` in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpagedattn.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "kv_append.hip", "decode.hip", "prefill.hip", "bench_util.hip", "block_manager.cpp"]

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed fp32 ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


DEBUG_LIB_PATH = os.path.join(PKG, "libpagedattn_debug.so")


def build(verbose: bool = False, jobs: int = 8, debug_checks: bool = True) -> str:
    """Compile every HIP source for gfx950 and link ``libpagedattn.so`` (and,
    with ``debug_checks``, ``libpagedattn_debug.so``: the same code built with
    PA_DEBUG_CHECKS, whose kernels trap on a broken device-side contract);
    returns the release library's path."""
    hipcc = _hipcc()
    variants = [(LIB_PATH, BUILD_DIR, [])]
    if debug_checks:
        variants.append((DEBUG_LIB_PATH, os.path.join(BUILD_DIR, "debug"), ["-DPA_DEBUG_CHECKS"]))
    cmds, links = [], []
    for lib_path, bdir, extra in variants:
        os.makedirs(bdir, exist_ok=True)
        objs = []
        for src in SOURCES:
            obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([hipcc, *CXXFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        links.append((lib_path, objs))
    with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    for lib_path, objs in links:
        tmp = lib_path + ".tmp"
        _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
