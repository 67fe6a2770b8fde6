"""KVSCORE_TRACE=1 logs one line per launch (kernel, grid, block, shape) to stderr.  The
flag is read once per process, so the check runs a small step in a child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STEP = r"""
import torch, compaction_kv_score_amd as kv, synth
dev = torch.device("cuda:0")
w = synth.workload("qwen2.5-1.5b-1layer-n512")
k, v, bt = synth.kv_cache(w, seed=0, device=dev, paged_shuffle=True, extra_pages=2)
q = synth.window_queries(w, seed=0, device=dev)
acc = torch.zeros(w.n_tokens, device=dev)
score = torch.zeros(w.n_tokens, device=dev)
pin = torch.zeros(w.n_tokens, dtype=torch.uint8, device=dev)
cache = kv.PagedCache(k, v, w.n_tokens, bt)
kv.kv_score(cache, q, policy="h2o", window=w.window, item_tokens=1, accum=acc, item_score=score, item_pinned=pin)
keep = torch.zeros(128, dtype=torch.int32, device=dev)
nk = torch.zeros(1, dtype=torch.int64, device=dev)
kv.kv_select(score, pin, 1, w.n_tokens, 128, keep, nk)
dk = torch.zeros((1, 8, 16, 2, 128), dtype=torch.bfloat16, device=dev)
pos = torch.arange(w.n_tokens, dtype=torch.int32, device=dev)
kv.kv_compact_rerope(cache, kv.PagedCache(dk, torch.zeros_like(dk), 128), keep, nk, 128, pos, None, renumber_base=0)
torch.cuda.synchronize()
print("step done")
"""


@pytest.mark.parametrize("flag,expect", [("1", True), ("0", False)])
def test_trace_logs_every_launch(flag, expect):
    env = dict(os.environ, KVSCORE_TRACE=flag)
    r = subprocess.run([sys.executable, "-c", STEP], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "step done" in r.stdout, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[kvscore] ")]
    if not expect:
        assert lines == []
        return
    names = [l.split()[1] for l in lines]
    # a grid this small combines the LSE inside the mass pass (no combine launch)
    assert names == ["lse_pass", "mass_pass", "epilogue", "select", "compact"], names
    assert "combines_lse" in lines[1]
    assert "tokens=512" in lines[0] and "block=" in lines[0] and "grid=" in lines[0]
    assert "stream_stores=0" in lines[-1]
