"""The host code of libkvscore (argument validation, workspace layout, RoPE tables, swap
bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host pass (device code unchanged) and
the C-ABI checks of test_abi.py run against it in a child process: the ASan runtime is
preloaded, Python allocates through malloc so that ctypes buffers are tracked, and any
report ends the run with an error.  The build is kept under _build/ and redone when a
source changes.
"""
import hashlib
import os
import subprocess
import sys

import pytest

from compaction_kv_score_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitized")


def _sources_hash():
    h = hashlib.sha256()
    for name in B.SOURCES + ["kv_internal.h"]:
        with open(os.path.join(B.CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(B.INCLUDE, "kvscore.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(B.HIPCC_FLAGS + B.SANITIZE_HOST_FLAGS).encode())
    return h.hexdigest()


@pytest.fixture(scope="module")
def sanitized_lib():
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("the ROCm compiler's ASan runtime is not installed")
    lib = os.path.join(OUT, "libkvscore_san.so")
    stamp = os.path.join(OUT, "sources.sha256")
    want = _sources_hash()
    if not (os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read() == want):
        B.build_sanitized(OUT)
        with open(stamp, "w") as f:
            f.write(want)
    return lib, rt


def test_abi_checks_clean_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ, KVSCORE_LIB=lib, LD_PRELOAD=rt, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
    # the child really loaded the sanitized build
    probe = subprocess.run([sys.executable, "-c", "import compaction_kv_score_amd as kv; print(kv.lib()._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
