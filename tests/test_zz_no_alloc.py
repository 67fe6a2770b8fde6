"""kv_select_noalloc (selection in the library's fixed device scratch) against kv_select
with a caller workspace: bit-identical keep lists, counts and status words, on calls in a
row whose sizes shrink, so the second call runs on the scratch the first one left."""
import pytest
import torch

import compaction_kv_score_amd as kv
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(n_items, item_tokens, n_tokens, budget, seed, pin_frac, alphabet=None, nan=0.0):
    s = synth.scores(n_items, seed=seed, alphabet=alphabet, nan_frac=nan, neg_zero=True).to(DEV)
    pin = synth.pinned_mask(n_items, seed=seed, frac=pin_frac).to(DEV) if pin_frac else None
    cap = min(n_tokens, budget * item_tokens + 64)
    out = []
    for fn in ("ws", "noalloc"):
        keep = torch.full((cap,), -1, dtype=torch.int32, device=DEV)
        nk = torch.full((1,), -1, dtype=torch.int64, device=DEV)
        st = torch.full((1,), 0x7777, dtype=torch.int32, device=DEV)
        if fn == "ws":
            kv.kv_select(s, pin, item_tokens, n_tokens, budget, keep, nk, st)
        else:
            kv.kv_select_noalloc(s, pin, item_tokens, n_tokens, budget, keep, nk, st)
        torch.cuda.synchronize()
        out.append((keep.cpu(), int(nk.item()), int(st.item())))
    (k0, n0, s0), (k1, n1, s1) = out
    assert n0 == n1 and s0 == s1 and torch.equal(k0, k1), (n_items, n0, n1, s0, s1)
    assert n0 > 0


def test_select_noalloc_matches_workspace_select_on_shrinking_calls():
    # token mode at the 100K-token budget, then a much smaller row with ties and NaNs
    _both(100_000, 1, 100_000, 2048, seed=1, pin_frac=0.0013)
    _both(5_000, 1, 5_000, 700, seed=2, pin_frac=0.02, alphabet=[1.0, 2.0, 3.0], nan=0.01)
    # page mode at 1M tokens, then a tiny row with a partial last page
    _both(62_500, 16, 1_000_000, 128, seed=3, pin_frac=0.001)
    _both(3, 16, 37, 2, seed=4, pin_frac=0.0)


def test_select_noalloc_in_a_graph():
    """The callers it is for include code under graph capture: captured after one eager
    call on the device, replayed four times with new scores, every replay equal to
    kv_select with a workspace on the same scores."""
    n, budget = 50_000, 2048
    score = torch.empty(n, device=DEV)
    pinned = synth.pinned_mask(n, seed=5, frac=0.001).to(DEV)
    keep = torch.zeros(budget, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    score.copy_(synth.scores(n, seed=6).to(DEV))
    kv.kv_select_noalloc(score, pinned, 1, n, budget, keep, nk, st)      # first call, outside capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kv.kv_select_noalloc(score, pinned, 1, n, budget, keep, nk, st)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kv.kv_select_noalloc(score, pinned, 1, n, budget, keep, nk, st)
    ref_keep = torch.zeros_like(keep)
    ref_nk = torch.zeros_like(nk)
    ref_st = torch.zeros_like(st)
    for rep in range(4):
        score.copy_(synth.scores(n, seed=20 + rep, alphabet=[1.0, 2.0, 3.0] if rep % 2 else None).to(DEV))
        keep.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kv.kv_select(score, pinned, 1, n, budget, ref_keep, ref_nk, ref_st)
        torch.cuda.synchronize()
        assert int(nk.item()) == int(ref_nk.item()) == budget and int(st.item()) == int(ref_st.item()), rep
        assert torch.equal(keep, ref_keep), rep
