"""The public header compiles as plain C99 and agrees with the Python binding.

A small C program is built with gcc against include/kvscore.h and linked with the
library; it prints the size and every field offset of each struct the ABI passes by
pointer, and every integer constant the header defines. Those must equal the ctypes
declarations and constants of the binding, so a field added on one side only (or a
padding difference) fails here rather than as a wrong value on the GPU.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import compaction_kv_score_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvscore.h")
ROCM_INC = "/opt/rocm/include"

STRUCTS = {
    "kv_cache_desc": kv.KvCacheDesc,
    "kv_meta_desc": kv.KvMetaDesc,
    "kv_score_params": kv.KvScoreParams,
    "kv_rope": kv.KvRope,
    "kv_ref_store": kv.KvRefStore,
}


def _header_constants():
    names = []
    with open(HEADER) as f:
        for line in f:
            m = re.match(r"#define (KV_[A-Z0-9_]+)\s+\S", line)
            if m:
                names.append(m.group(1))
    return names


def _program(consts):
    out = ["#include <stdio.h>", "#include <stddef.h>", '#include "kvscore.h"',
           "int main(void) {"]
    for cname, cls in STRUCTS.items():
        out.append(f'  printf("size {cname} %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            out.append(f'  printf("off {cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    for c in consts:
        out.append(f'  printf("const {c} %lld\\n", (long long)({c}));')
    out.append('  printf("abi %d\\n", kv_abi_version());')
    out.append("  return 0;\n}")
    return "\n".join(out) + "\n"


@pytest.fixture(scope="module")
def c_report(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("gcc or the ROCm headers are not available")
    libdir = os.path.dirname(kv.lib()._name)
    consts = _header_constants()
    d = tmp_path_factory.mktemp("hdr")
    src = d / "probe.c"
    exe = d / "probe"
    src.write_text(_program(consts))
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.dirname(HEADER)}", f"-isystem{ROCM_INC}",
           str(src), f"-L{libdir}", "-lkvscore", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    rep = {}
    for line in r.stdout.splitlines():
        kind, key, val = line.split() if line.count(" ") == 2 else (line.split()[0], "", line.split()[1])
        rep[(kind, key)] = int(val)
    return consts, rep


def test_struct_layouts_match_binding(c_report):
    _, rep = c_report
    for cname, cls in STRUCTS.items():
        assert rep[("size", cname)] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert rep[("off", f"{cname}.{fname}")] == getattr(cls, fname).offset, (cname, fname)


def test_header_constants_match_binding(c_report):
    consts, rep = c_report
    assert len(consts) >= 20
    for c in consts:
        assert hasattr(kv, c), f"{c} is defined in the header but not in the binding"
        assert getattr(kv, c) == rep[("const", c)], c


def test_abi_version_from_c(c_report):
    _, rep = c_report
    assert rep[("abi", "")] == kv.KV_ABI_VERSION
