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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (device code is compiled as
# usual; every sanitizer flag applies to the host pass only).
SANITIZE_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm compiler (to LD_PRELOAD into a
    process that loads the sanitized library), or '' when it is not installed."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Compile libkvscore with the host code under ASan and UBSan into out_dir (for the
    host-side checks of the argument validation and bookkeeping); returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-O3")] + ["-O1", "-g"] + SANITIZE_HOST_FLAGS
    from concurrent.futures import ThreadPoolExecutor
    objs = [os.path.join(out_dir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc(), *flags, "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1, 8))) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    lib = os.path.join(out_dir, "libkvscore_san.so")
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *SANITIZE_HOST_FLAGS, "-shared-libasan", *objs,
          "-o", lib], verbose)
    for o in objs:
        os.remove(o)
    return lib


C_PIPELINE_SRC = os.path.join(ROOT, "tests", "c_pipeline.c")
C_PIPELINE = os.path.join(ROOT, "tests", "c_pipeline")


def build_c_pipeline(verbose: bool = False) -> str:
    """Build the C test program that drives the library through include/kvscore.h alone
    (plain C99 host code, gcc), next to its source; it finds libkvscore.so relative to
    itself.  Returns its path."""
    libdir = os.path.dirname(LIB)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_PIPELINE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-isystem", os.path.join(rocm, "include"), C_PIPELINE_SRC,
           "-L", libdir, "-lkvscore", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../compaction_kv_score_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, C_PIPELINE)
    return C_PIPELINE


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_pipeline(verbose=True))
