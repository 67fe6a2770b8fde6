"""The C ABI driven by a C program with no Python between caller and library.

tests/c_pipeline.c includes only include/kvscore.h and the HIP runtime header, loads
seeded inputs from files, runs one eviction step (H2O + foresight scoring with pinned
sinks and recent tokens, token selection, compaction with renumbering) on a stream of its
own and writes the outputs back.  They are held to the same bars as the parity tests:
mass and scores within 1e-5 relative of the oracle, the keep list equal to the oracle's
selection on the device's own scores, V bit-exact, re-rotated K within 1 bf16 ulp."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
import synth

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_pipeline.c")
EXE = os.path.join(ROOT, "tests", "c_pipeline")
RTOL = 1e-5


def _program():
    """The program built by __graft_entry__.build(), rebuilt with gcc (host code only, about
    a second) when it is missing or older than its source or the library."""
    lib = kv.LIB_PATH
    if os.path.exists(EXE) and os.path.getmtime(EXE) >= max(os.path.getmtime(SRC), os.path.getmtime(lib)):
        return EXE
    from compaction_kv_score_amd.build import build_c_pipeline
    if shutil.which("gcc") is None:
        pytest.fail("gcc is needed to build tests/c_pipeline")
    return build_c_pipeline()


def _ulp_bf16(x):
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(x)
    return np.where(x == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def _bf16_file(path, shape):
    raw = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return raw.view(np.float32).astype(np.float64).reshape(shape)


def test_c_program_runs_one_step(tmp_path):
    w = synth.workload("qwen3-8b-n100k", n_tokens=3000, n_layers=2, n_spans=40, budget_tokens=512)
    L, HKV, HQ, N, W, B = w.n_layers, w.n_kv_heads, w.n_q_heads, w.n_tokens, w.window, w.budget_tokens
    k, v, bt = synth.kv_cache(w, seed=21, device="cpu")
    assert bt is None
    q = synth.window_queries(w, seed=21)
    sid, sbonus = synth.spans(w, seed=21, p_needed=0.2)
    src, out = tmp_path / "in", tmp_path / "out"
    src.mkdir()
    out.mkdir()
    for name, t in (("k", k), ("v", v), ("q", q)):
        t.contiguous().view(torch.int16).numpy().tofile(src / f"{name}.bin")
    sid.numpy().astype(np.int32).tofile(src / "span_id.bin")
    sbonus.numpy().astype(np.float32).tofile(src / "span_bonus.bin")
    (src / "meta.txt").write_text(f"{L} {HKV} {HQ} {N} {W} {B} {w.n_spans} {w.n_sink} {w.n_recent} "
                                  f"{w.limit} {w.rope_theta!r}\n")
    print(f"c_pipeline: N={N} L={L} B={B}", flush=True)
    r = subprocess.run([_program(), str(src), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    mass = np.fromfile(out / "mass.bin", dtype=np.float32).astype(np.float64)
    score = np.fromfile(out / "item_score.bin", dtype=np.float32).astype(np.float64)
    pinned = np.fromfile(out / "item_pinned.bin", dtype=np.uint8).astype(bool)
    keep = np.fromfile(out / "keep.bin", dtype=np.int32).astype(np.int64)
    n_keep = int(np.fromfile(out / "n_keep.bin", dtype=np.int64)[0])
    status = int(np.fromfile(out / "status.bin", dtype=np.uint32)[0])
    new_pos = np.fromfile(out / "new_pos.bin", dtype=np.int32)
    dk = _bf16_file(out / "dst_k.bin", (L, B, HKV, 128))
    dv = _bf16_file(out / "dst_v.bin", (L, B, HKV, 128))

    kl = k.float().double().numpy().reshape(L, -1, HKV, 128)[:, :N]
    vl = v.float().double().numpy().reshape(L, -1, HKV, 128)[:, :N]
    ref = O.score_step(q.float().double().numpy(), kl, policy="h2o", accum=np.zeros(N), span_id=sid.numpy(),
                       span_bonus=sbonus.numpy(), n_sink=w.n_sink, n_recent=w.n_recent)
    for got, want, what in ((mass, ref["mass"], "mass"), (score, ref["item_score"], "score")):
        bad = np.abs(got - want) > RTOL * np.abs(want) + 1e-35
        assert not bad.any(), (what, int(bad.sum()))
    assert (pinned == ref["item_pinned"]).all()
    assert (np.asarray(sbonus) > 0).any() and pinned.sum() == w.n_sink + w.n_recent
    want_keep, st = O.select_items(score, pinned, B)
    assert n_keep == B and status == 0 and st == 0
    assert (keep == want_keep).all()
    rk, rv, rpos = O.compact_rerope(kl, vl, keep, np.arange(N), 0, w.rope_theta)
    assert (new_pos == rpos).all() and (rpos == np.arange(B)).all()
    assert (dv == rv).all()
    assert (np.abs(dk - rk) <= _ulp_bf16(rk)).all()
