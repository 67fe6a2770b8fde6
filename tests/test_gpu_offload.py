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


@pytest.mark.parametrize("n,n_keep,chunk,shuffle", [(3000, 2048, 1024, True), (1500, 100, 256, True),
                                                    (700, 650, 16, False), (4096, 0, 1000, True)])
def test_load_rows_restores_offloaded_rows(n, n_keep, chunk, shuffle):
    """Offload the rows a compaction drops, blank them, load them back into the slots they
    came from (with their positions as metadata): the cache equals the original and the
    oracle's load_rows of the host rows, bit for bit."""
    nl, hkv = 3, 2
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=n + 7, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    k0, v0 = _logical(k, bt, n), _logical(v, bt, n)
    rng = np.random.default_rng(n + 2)
    keep = np.sort(rng.choice(n, n_keep, replace=False))
    ev = O.evicted_tokens(n, keep)
    hk = torch.zeros((nl, len(ev), hkv, 128), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.zeros_like(hk).pin_memory()
    ht = torch.full((len(ev),), -1, dtype=torch.int32, pin_memory=True)
    cache = kv.PagedCache(k, v, n, bt)
    keep_d = torch.from_numpy(keep.astype(np.int32)).to(DEV) if n_keep else None
    kv.kv_offload_evicted(cache, keep_d, n_keep, hk, hv, ht, chunk=chunk)
    torch.cuda.synchronize()
    # blank the evicted slots through a load of zeros, then load the offloaded rows back
    slots = ht.to(DEV)
    zk = torch.zeros_like(hk).pin_memory()
    kv.kv_load_rows(cache, slots, zk, zk, chunk=chunk)
    torch.cuda.synchronize()
    blank_k = _logical(k, bt, n)
    assert (blank_k[:, ev] == 0).all() and (blank_k[:, keep] == k0[:, keep]).all()
    pos_src = torch.from_numpy((ev * 3 + 11).astype(np.int32)).to(DEV)
    pos = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    kv.kv_load_rows(cache, slots, hk, hv, chunk=chunk, meta=[(pos_src, pos)])
    torch.cuda.synchronize()
    want_k = O.load_rows(blank_k, ev, hk.double().numpy())
    assert (_logical(k, bt, n) == want_k).all() and (want_k == k0).all()
    assert (_logical(v, bt, n) == v0).all()
    p = pos.cpu().numpy()
    assert (p[ev] == ev * 3 + 11).all() and (p[keep] == -1).all()


def test_load_rows_subrange_and_skipped_slots():
    """Rows [host_first, host_first + count) of a larger pool; slots outside the row are
    skipped by the kernel's bounds check."""
    nl, hkv, n = 2, 4, 500
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=3, device=DEV, paged_shuffle=True, extra_pages=1)
    before = _logical(k, bt, n)
    rng = np.random.default_rng(9)
    pool = O.bf16_round(rng.standard_normal((nl, 300, hkv, 128)))
    hk = torch.from_numpy(pool).to(torch.bfloat16).pin_memory()
    hv = (-hk).pin_memory()
    slots = rng.choice(n, 120, replace=False).astype(np.int32)
    slots[[5, 77]] = [n + 3, -1]
    kv.kv_load_rows(kv.PagedCache(k, v, n, bt), torch.from_numpy(slots).to(DEV), hk, hv, host_first=150,
                    chunk=50)
    torch.cuda.synchronize()
    ok = np.ones(120, bool)
    ok[[5, 77]] = False
    want = O.load_rows(before, slots[ok], pool[:, 150:270][:, ok])
    assert (_logical(k, bt, n) == want).all()
    assert (_logical(v, bt, n)[:, slots[ok]] == -pool[:, 150:270][:, ok]).all()


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("count,chunk,in_first,buf_first,shuffle", [
    (700, 256, 0, 900, True),        # ragged last chunk
    (1024, 1024, 50, 1100, True),    # one chunk
    (2000, 1024, 2000, 0, False),    # buffer before the incoming rows
    (33, 8, 40, 0, True),
    (3000, 128, 100, 3200, True),    # 24 chunks: the two directions overlap many times
])
def test_swap_chunked_parity(count, chunk, in_first, buf_first, shuffle, two_streams):
    """Penelope's both-tiers-full swap through the CPU buffer against the oracle: GPU slots,
    every pool row, where each outgoing row landed and the next buffer; on one stream, and
    with the incoming side on a second stream."""
    nl, hkv, n = 3, 2, 4000
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=count, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    k0, v0 = _logical(k, bt, n), _logical(v, bt, n)
    rng = np.random.default_rng(count + chunk)
    rows = max(in_first + count, buf_first + min(chunk, count)) + 17
    pk = O.bf16_round(rng.standard_normal((nl, rows, hkv, 128)))
    pv = O.bf16_round(rng.standard_normal((nl, rows, hkv, 128)))
    hk = torch.from_numpy(pk).to(torch.bfloat16).pin_memory()
    hv = torch.from_numpy(pv).to(torch.bfloat16).pin_memory()
    slots = rng.choice(n, count, replace=False)
    in_stream = torch.cuda.Stream() if two_streams else None
    slots_d = torch.from_numpy(slots.astype(np.int32)).to(DEV)
    torch.cuda.synchronize()
    out_rows, nxt, _ = kv.kv_swap_chunked(kv.PagedCache(k, v, n, bt), slots_d, hk, hv, in_first, buf_first,
                                          chunk=chunk, in_stream=in_stream)
    torch.cuda.current_stream().synchronize()         # the call completes on the current stream
    gk, pk2, want_rows, want_next = O.chunked_swap(k0, pk, slots, in_first, buf_first, chunk)
    gv, pv2, _, _ = O.chunked_swap(v0, pv, slots, in_first, buf_first, chunk)
    assert out_rows == want_rows.tolist() and nxt == want_next
    assert (_logical(k, bt, n) == gk).all() and (_logical(v, bt, n) == gv).all()
    assert (hk.double().numpy() == pk2).all() and (hv.double().numpy() == pv2).all()
