"""The launch sequences contain no memset and allocate nothing, so a caller can capture
them in a HIP graph.  Each test captures one sequence, replays it several times with
eager work and synchronisations between the replays, and checks every replay against
the eager result of the same inputs."""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_select_and_compact_in_a_graph():
    w = synth.workload("qwen3-8b-n100k", n_tokens=20_000, n_layers=4)
    k, v, _ = synth.kv_cache(w, seed=3, device=DEV)
    N, B = w.n_tokens, w.budget_tokens
    score = torch.empty(N, device=DEV)
    pinned = torch.zeros(N, dtype=torch.uint8, device=DEV)
    pinned[:4] = 1
    keep = torch.zeros(B, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(kv.kv_select_workspace_size(N), dtype=torch.uint8, device=DEV)
    dk = torch.zeros((4, B // 16, 16, 8, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    newp = torch.zeros(B, dtype=torch.int32, device=DEV)
    src, dst = kv.PagedCache(k, v, N), kv.PagedCache(dk, dv, B)

    def seq():
        kv.kv_select(score, pinned, 1, N, B, keep, nk, status, workspace=ws)
        kv.kv_compact_rerope(src, dst, keep, nk, B, pos, newp, renumber_base=0, rope_theta=1e6, limit=8192)

    score.copy_(torch.from_numpy(synth.scores(N, seed=1).numpy()).to(DEV))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for rep in range(4):
        score.copy_(torch.from_numpy(synth.scores(N, seed=10 + rep).numpy()).to(DEV))
        dk.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (keep.clone(), int(nk.item()), dk.clone(), newp.clone())
        dk.zero_()
        seq()                                   # eager, same inputs
        torch.cuda.synchronize()
        assert int(nk.item()) == got[1] == B and int(status.item()) == 0, rep
        assert torch.equal(keep, got[0]) and torch.equal(dk, got[2]) and torch.equal(newp, got[3]), rep


def test_lrfu_in_a_graph():
    n = 70_000
    att = torch.empty(n, device=DEV)
    ks = torch.zeros(n, device=DEV)
    hit = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ws = torch.empty(kv.kv_lrfu_workspace_size(n), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(2)
    att.copy_(torch.from_numpy((rng.random(n) ** 6).astype(np.float32)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kv.kv_lrfu_update(att, ks, top_p=0.9, decay=0.5, hit=hit, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kv.kv_lrfu_update(att, ks, top_p=0.9, decay=0.5, hit=hit, workspace=ws)
    for rep in range(4):
        att.copy_(torch.from_numpy((rng.random(n) ** 6).astype(np.float32)))
        ks0 = torch.from_numpy(rng.random(n).astype(np.float32)).to(DEV)
        ks.copy_(ks0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_ks, got_hit = ks.clone(), hit.clone()
        ks.copy_(ks0)
        kv.kv_lrfu_update(att, ks, top_p=0.9, decay=0.5, hit=hit, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got_ks, ks) and torch.equal(got_hit, hit), rep


def test_score_in_a_graph():
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=8000, window=64, n_q_heads=32, n_kv_heads=8, n_layers=2)
    k, v, bt = synth.kv_cache(w, seed=4, device=DEV, paged_shuffle=True, extra_pages=1)
    q = synth.window_queries(w, seed=4, device=DEV)
    N = w.n_tokens
    acc = torch.zeros(N, device=DEV)
    out = dict(mass=torch.zeros(N, device=DEV), item_score=torch.zeros(N, device=DEV),
               item_pinned=torch.zeros(N, dtype=torch.uint8, device=DEV))
    cache = kv.PagedCache(k, v, N, bt)
    kw = dict(policy="h2o", window=w.window, item_tokens=1, accum=acc, **out)
    ws = torch.empty(kv.kv_score_workspace_size(cache, q, **kw), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kv.kv_score(cache, q, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kv.kv_score(cache, q, workspace=ws, **kw)
    for rep in range(3):
        q.copy_(synth.window_queries(w, seed=20 + rep, device=DEV))
        acc.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in out.items()}
        acc.zero_()
        kv.kv_score(cache, q, workspace=ws, **kw)
        torch.cuda.synchronize()
        for key in out:
            assert torch.equal(got[key], out[key]), (rep, key)


def test_memdecay_page_step_in_a_graph():
    """MemDecay page scoring, page selection and compaction with renumbering (the
    Qwen2.5-1.5B-shaped step: 28 layers, N = 2,048, budget 512 tokens) captured as one
    graph; each replay matches the eager step on the same state bit for bit."""
    w = synth.workload("qwen2.5-1.5b-n2048")
    N, pg, B = w.n_tokens, w.page_size, w.budget_tokens
    k, v, bt = synth.kv_cache(w, seed=5, device=DEV, paged_shuffle=True, extra_pages=2)
    q = synth.window_queries(w, seed=5, device=DEV)
    ewma0, clock0 = (t.to(DEV) for t in synth.memdecay_state(w, seed=5))
    ewma, clock = ewma0.clone(), clock0.clone()
    b_r, lam = synth.region_params(5)
    n_items = w.n_pages
    item_score = torch.zeros(n_items, device=DEV)
    item_pinned = torch.zeros(n_items, dtype=torch.uint8, device=DEV)
    src = kv.PagedCache(k, v, N, bt)
    kw = dict(policy="memdecay", window=w.window, item_tokens=pg, region=synth.regions(w, seed=5).to(DEV),
              base_prio=b_r.to(DEV), decay_rate=lam.to(DEV), rho=w.rho, alpha=w.alpha, tau=w.tau, dt_steps=1,
              ewma=ewma, clock=clock, pinned_regions=1, item_score=item_score, item_pinned=item_pinned)
    ws = torch.empty(kv.kv_score_workspace_size(src, q, **kw), dtype=torch.uint8, device=DEV)
    ws_sel = torch.empty(kv.kv_select_workspace_size(n_items), dtype=torch.uint8, device=DEV)
    keep = torch.zeros(B, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dk = torch.zeros((w.n_layers, B // pg, pg, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    dst = kv.PagedCache(dk, dv, B)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    newp = torch.zeros(B, dtype=torch.int32, device=DEV)
    outs = (item_score, item_pinned, ewma, clock, keep, nk, status, dk, dv, newp)

    def step():
        kv.kv_score(src, q, workspace=ws, **kw)
        kv.kv_select(item_score, item_pinned, pg, N, w.budget_items, keep, nk, status, workspace=ws_sel)
        kv.kv_compact_rerope(src, dst, keep, nk, B, pos, newp, renumber_base=0, rope_theta=w.rope_theta)

    def clear():
        for t in (item_score, item_pinned, keep, nk, dk, dv, newp):
            t.zero_()
        status.fill_(7)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        q.copy_(synth.window_queries(w, seed=30 + rep, device=DEV))
        clear()
        ewma.copy_(ewma0)
        clock.copy_(clock0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        clear()
        ewma.copy_(ewma0)
        clock.copy_(clock0)
        step()                                  # eager, same inputs and state
        torch.cuda.synchronize()
        assert int(nk.item()) == B and int(status.item()) == 0, rep
        for i, (x, y) in enumerate(zip(got, outs)):
            assert torch.equal(x, y), (rep, i)
