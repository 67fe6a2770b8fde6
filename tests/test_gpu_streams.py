"""Calls on different streams are independent when their buffers (workspaces included)
are disjoint: two score -> select -> compact pipelines enqueued on two streams at the
same time give the same bits as each one run alone on the default stream."""
import pytest
import torch

import compaction_kv_score_amd as kv
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class _Pipeline:
    """One row's H2O + foresight scoring, token selection and compaction with
    renumbering, with every buffer and workspace of its own."""

    def __init__(self, w, seed):
        self.w = w
        N, B, NL = w.n_tokens, w.budget_tokens, w.n_layers
        k, v, _ = synth.kv_cache(w, seed=seed, device=DEV)
        self.q = synth.window_queries(w, seed=seed, device=DEV)
        sid, bonus = synth.spans(w, seed=seed, p_needed=0.05)
        self.sid, self.bonus = sid.to(DEV), bonus.to(DEV)
        self.acc = torch.zeros(N, device=DEV)
        self.item_score = torch.zeros(N, device=DEV)
        self.item_pinned = torch.zeros(N, dtype=torch.uint8, device=DEV)
        self.keep = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.nk = torch.zeros(1, dtype=torch.int64, device=DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.pos = torch.arange(N, dtype=torch.int32, device=DEV)
        self.newp = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.dk = torch.zeros((NL, B // 16, 16, w.n_kv_heads, 128), dtype=torch.bfloat16, device=DEV)
        self.dv = torch.zeros_like(self.dk)
        self.src = kv.PagedCache(k, v, N)
        self.dst = kv.PagedCache(self.dk, self.dv, B)
        self.kw = dict(policy="h2o", window=w.window, item_tokens=1, accum=self.acc, span_id=self.sid,
                       span_bonus=self.bonus, n_sink=w.n_sink, n_recent=w.n_recent,
                       item_score=self.item_score, item_pinned=self.item_pinned)
        self.ws = torch.empty(kv.kv_score_workspace_size(self.src, self.q, **self.kw), dtype=torch.uint8,
                              device=DEV)
        self.ws_sel = torch.empty(kv.kv_select_workspace_size(N), dtype=torch.uint8, device=DEV)

    def clear(self):
        for t in (self.item_score, self.item_pinned, self.keep, self.nk, self.newp, self.dk, self.dv):
            t.zero_()
        self.status.fill_(7)

    def run(self):
        """Enqueue the pipeline on the current stream (the accumulator starts at zero)."""
        w = self.w
        self.acc.zero_()
        kv.kv_score(self.src, self.q, workspace=self.ws, **self.kw)
        kv.kv_select(self.item_score, self.item_pinned, 1, w.n_tokens, w.budget_tokens, self.keep, self.nk,
                     self.status, workspace=self.ws_sel)
        kv.kv_compact_rerope(self.src, self.dst, self.keep, self.nk, w.budget_tokens, self.pos, self.newp,
                             renumber_base=0, rope_theta=w.rope_theta, limit=w.limit)

    def outputs(self):
        return [t.clone() for t in (self.acc, self.item_score, self.item_pinned, self.keep, self.nk,
                                    self.status, self.newp, self.dk, self.dv)]


def test_two_pipelines_on_two_streams():
    w = synth.workload("qwen3-8b-n100k", n_tokens=30_000, n_layers=4)
    a, b = _Pipeline(w, 1), _Pipeline(w, 2)
    # alone, one after the other on the default stream
    a.clear()
    b.clear()
    a.run()
    torch.cuda.synchronize()
    b.run()
    torch.cuda.synchronize()
    ref_a, ref_b = a.outputs(), b.outputs()
    assert int(ref_a[4].item()) == w.budget_tokens and int(ref_a[5].item()) == 0
    assert not torch.equal(ref_a[3], ref_b[3])          # different rows select differently
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        a.clear()
        b.clear()
        torch.cuda.synchronize()
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            a.run()
        with torch.cuda.stream(sb):
            b.run()
        torch.cuda.synchronize()
        for got, want in ((a.outputs(), ref_a), (b.outputs(), ref_b)):
            for i, (x, y) in enumerate(zip(got, want)):
                assert torch.equal(x, y), (rep, i)
