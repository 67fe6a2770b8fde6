"""Build libkvscore.so (gfx950 only) in place with hipcc.

Usage: python -m compaction_kv_score_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvscore.so")

SOURCES = ["kv_api.hip", "kv_score.hip", "kv_epilogue.hip", "kv_select.hip", "kv_compact.hip",
           "kv_lrfu.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-pass-failed",
    # packed fp32 vector ops stay disabled: only scalar fp32 VALU code is generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link libkvscore.so next
    to this file; returns its path."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="kvscore_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc(), *compile_flags, "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
