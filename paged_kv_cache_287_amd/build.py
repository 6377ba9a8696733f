"""Compile the HIP sources under csrc/ for gfx950 into the in-tree shared library libpa.so.

Usage: ``python paged_kv_cache_287_amd/build.py`` (run by path: importing the package itself
requires the built library), or ``build()`` from ``__graft_entry__``.
Every call recompiles. Objects go to ``_build/`` next to this file; the library lands next to
this file so that the binding (and anything copying the source tree) finds it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.hip", "decode.hip", "decode_mfma.hip", "merge.hip", "prefill_mfma.hip", "cache_ops.hip",
           "probe.hip"]

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return proc.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link libpa.so. Returns the library path; raises on failure."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            print(" ".join(cmd))
            if out:
                print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed for {cmd[-3]}")
    tmp = LIB_PATH + ".tmp"
    # no RPATH: libamdhip64.so.7 resolves to the runtime already loaded by torch
    link = [CLANGXX, "-shared", "-fPIC", "-o", tmp, *objs, f"-L{ROCM}/lib", "-lamdhip64"]
    rc, out = _run(link)
    if verbose or rc != 0:
        print(" ".join(link))
        if out:
            print(out)
    if rc != 0:
        raise RuntimeError("link of libpa.so failed")
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
