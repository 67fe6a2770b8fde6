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
