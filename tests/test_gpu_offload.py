"""GPU parity of the evicted-row gather and the offload to pinned host memory
(kv_gather_evicted, kv_offload_evicted) against the oracle's complement of the keep
list.  Copies of bf16 data and token indices: bit-exact."""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
from layout import unpage
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _logical(t, bt, n):
    return unpage(t.float().cpu().double().numpy(), None if bt is None else bt.cpu().numpy(), 16, n)


@pytest.mark.parametrize("nl,hkv,n,n_keep,first,count,shuffle", [
    (2, 2, 1000, 300, 0, 700, True),
    (3, 8, 777, 0, 10, 500, False),
    (2, 2, 4096, 4000, 0, 96, True),
    (1, 4, 513, 512, 0, 1, True),
    (9, 4, 2000, 1500, 100, 400, True),     # 576 chunk pairs per token: three workgroups each
])
def test_gather_evicted_parity(nl, hkv, n, n_keep, first, count, shuffle):
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=n + n_keep, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    rng = np.random.default_rng(n)
    keep = np.sort(rng.choice(n, n_keep, replace=False))
    ev = O.evicted_tokens(n, keep)[first:first + count]
    pos = torch.from_numpy(rng.integers(0, 2 ** 31 - 1, n).astype(np.int32)).to(DEV)
    pages = -(-count // 16)
    dk = torch.zeros((nl, pages, 16, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    ids = torch.full((count,), -1, dtype=torch.int32, device=DEV)
    pos_out = torch.zeros(count, dtype=torch.int32, device=DEV)
    kv.kv_gather_evicted(kv.PagedCache(k, v, n, bt), torch.from_numpy(keep.astype(np.int32)).to(DEV), n_keep,
                         first, count, kv.PagedCache(dk, dv, count), ids, meta=[(pos, pos_out)])
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == ev).all()
    assert (_logical(dk, None, count) == _logical(k, bt, n)[:, ev]).all()
    assert (_logical(dv, None, count) == _logical(v, bt, n)[:, ev]).all()
    assert (pos_out.cpu().numpy() == pos.cpu().numpy()[ev]).all()


@pytest.mark.parametrize("n,n_keep,chunk", [(3000, 2048, 1024), (5000, 100, 1024), (700, 0, 256), (2048, 2048, 64)])
def test_offload_evicted_to_pinned_host(n, n_keep, chunk):
    nl, hkv = 3, 2
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=n, device=DEV, paged_shuffle=True, extra_pages=1)
    rng = np.random.default_rng(n + 1)
    keep = np.sort(rng.choice(n, n_keep, replace=False))
    ev = O.evicted_tokens(n, keep)
    n_ev = len(ev)
    hk = torch.zeros((nl, max(n_ev, 1), hkv, 128), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.zeros_like(hk).pin_memory()
    ht = torch.full((max(n_ev, 1),), -1, dtype=torch.int32, pin_memory=True)
    kv.kv_offload_evicted(kv.PagedCache(k, v, n, bt), torch.from_numpy(keep.astype(np.int32)).to(DEV)
                          if n_keep else None, n_keep, hk, hv, ht, chunk=chunk)
    torch.cuda.synchronize()
    if n_ev == 0:
        assert (ht == -1).all()
        return
    assert (ht.numpy() == ev).all()
    assert (hk.double().numpy() == _logical(k, bt, n)[:, ev]).all()
    assert (hv.double().numpy() == _logical(v, bt, n)[:, ev]).all()
