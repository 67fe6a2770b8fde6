"""Page-table segment eviction (kv_compact_segment_remap) against the oracle.

The surviving suffix is relinked in a new block table instead of moved, so the row read
through the new table must equal the oracle's compaction of the kept tokens (V and
unrotated K bit-exact, re-rotated K within 1 bf16 ulp), while physically nothing but the
re-rotated keys changes: every V page and every key whose position is kept stay
bit-identical in place.  The freed-page list is the evicted segment's pages."""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
import synth
from layout import unpage
from test_gpu_parity import assert_bf16_within_1ulp, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(nl, hkv, n, prefix, evict, base, theta, seed, meta=True, pg=16):
    w = synth.workload("mistral-7b-n131072-segment", n_layers=nl, n_kv_heads=hkv, n_q_heads=4 * hkv, n_tokens=n,
                       page_size=pg)
    k, v, bt = synth.kv_cache(w, seed=seed, device=DEV, paged_shuffle=True, extra_pages=3)
    k0, v0 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(seed)
    old_pos = (torch.arange(n, dtype=torch.int32) + torch.randint(0, 50, (1,), generator=g).int()).to(DEV)
    n_keep = n - evict
    keep_pages = -(-n_keep // pg)
    bt_out = torch.full((keep_pages + 2,), -7, dtype=torch.int32, device=DEV)
    freed = torch.full((evict // pg + 2,), -7, dtype=torch.int32, device=DEV)
    new_pos = torch.full((n_keep + 3,), -7, dtype=torch.int32, device=DEV)
    region = torch.randint(0, 7, (n,), generator=g, dtype=torch.int32).to(torch.uint8).to(DEV)
    span = torch.randint(-1, 200, (n,), generator=g, dtype=torch.int32).to(DEV)
    reg_out = torch.zeros(n_keep, dtype=torch.uint8, device=DEV)
    span_out = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
    kv.kv_compact_segment_remap(kv.PagedCache(k, v, n, bt), prefix, evict, bt_out, old_pos, new_pos,
                                freed_pages=freed, renumber_base=base, rope_theta=theta,
                                meta=[(region, reg_out), (span, span_out)] if meta else None)
    torch.cuda.synchronize()

    btn, bto = bt.cpu().numpy(), bt_out.cpu().numpy()
    pp, ep = prefix // pg, evict // pg
    want_bt = np.concatenate([btn[:pp], btn[pp + ep:]])
    assert (bto[:keep_pages] == want_bt).all() and (bto[keep_pages:] == -7).all()
    assert (freed.cpu().numpy()[:ep] == btn[pp:pp + ep]).all() and (freed.cpu().numpy()[ep:] == -7).all()

    keep = np.concatenate([np.arange(prefix), np.arange(prefix + evict, n)]).astype(np.int64)
    op = old_pos.cpu().numpy()
    kl = unpage(np64(k0), btn, pg, n)
    vl = unpage(np64(v0), btn, pg, n)
    rk, rv, rpos = O.compact_rerope(kl, vl, keep, op, base, theta)
    assert (new_pos.cpu().numpy()[:n_keep] == rpos).all() and (new_pos.cpu().numpy()[n_keep:] == -7).all()
    gk = unpage(np64(k), bto[:keep_pages], pg, n_keep)
    gv = unpage(np64(v), bto[:keep_pages], pg, n_keep)
    assert (gv == rv).all()
    same = rpos == op[keep]
    assert (gk[:, same] == rk[:, same]).all()
    assert_bf16_within_1ulp(gk, rk, "remapped K")
    # physically: V untouched everywhere, K untouched except the re-rotated keys
    assert torch.equal(v, v0)
    kphys, k0phys = np64(k), np64(k0)
    moved_phys = np.zeros(kphys.shape[1:3], bool)               # [physical page][slot]
    for r in np.nonzero(~same)[0]:
        j = keep[r]
        moved_phys[btn[j // pg], j % pg] = True
    assert (kphys[:, ~moved_phys] == k0phys[:, ~moved_phys]).all()
    if meta:
        assert (reg_out.cpu().numpy() == region.cpu().numpy()[keep]).all()
        assert (span_out.cpu().numpy() == span.cpu().numpy()[keep]).all()
    return int((~same).sum())


@pytest.mark.parametrize("nl,hkv,n,prefix,evict,base,theta", [
    (2, 8, 3000, 320, 960, 0, 1e4),       # renumbered: the suffix rotates by -E'; ragged last page
    (2, 8, 3000, 320, 960, -1, 1e4),      # positions kept (Penelope): nothing but the table changes
    (3, 2, 2048, 0, 512, 7, 1e6),         # no prefix; renumbered from base 7: every key rotates
    (1, 4, 1000, 496, 0, 0, 1e4),         # nothing evicted
    (2, 8, 1600, 1024, 576, 0, 1e4),      # everything after the prefix evicted
])
def test_segment_remap_parity(nl, hkv, n, prefix, evict, base, theta):
    rotated = _case(nl, hkv, n, prefix, evict, base, theta, seed=n + prefix)
    if base < 0:
        assert rotated == 0


def test_segment_remap_agrees_with_inplace():
    """The same eviction done by moving the suffix (kv_compact_segment_inplace) gives the
    same logical row bit for bit."""
    w = synth.workload("mistral-7b-n131072-segment", n_layers=2, n_tokens=5000)
    n, prefix, evict = w.n_tokens, 1024, 1504
    k, v, bt = synth.kv_cache(w, seed=9, device=DEV, paged_shuffle=True, extra_pages=2)
    k2, v2 = k.clone(), v.clone()
    pos = torch.arange(n, dtype=torch.int32, device=DEV)
    kv.kv_compact_segment_inplace(kv.PagedCache(k2, v2, n, bt), prefix, evict, pos, renumber_base=0,
                                  rope_theta=w.rope_theta)
    bt_out = torch.zeros(-(-(n - evict) // 16), dtype=torch.int32, device=DEV)
    new_pos = torch.zeros(n - evict, dtype=torch.int32, device=DEV)
    kv.kv_compact_segment_remap(kv.PagedCache(k, v, n, bt), prefix, evict, bt_out,
                                torch.arange(n, dtype=torch.int32, device=DEV), new_pos, renumber_base=0,
                                rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    n_keep = n - evict
    assert torch.equal(new_pos, pos[:n_keep])
    btn = bt.cpu().numpy()
    a_k = unpage(np64(k2), btn, 16, n_keep)
    a_v = unpage(np64(v2), btn, 16, n_keep)
    b_k = unpage(np64(k), bt_out.cpu().numpy(), 16, n_keep)
    b_v = unpage(np64(v), bt_out.cpu().numpy(), 16, n_keep)
    assert (a_k == b_k).all() and (a_v == b_v).all()


def test_segment_remap_rejects_unaligned_and_overlapping():
    w = synth.workload("mistral-7b-n131072-segment", n_layers=1, n_tokens=512)
    k, v, bt = synth.kv_cache(w, seed=1, device=DEV, paged_shuffle=True)
    c = kv.PagedCache(k, v, 512, bt)
    pos = torch.arange(512, dtype=torch.int32, device=DEV)
    out = torch.zeros(32, dtype=torch.int32, device=DEV)
    npos = torch.zeros(512, dtype=torch.int32, device=DEV)
    bt0 = bt.clone()
    cases = [(16, 40, out, npos), (8, 32, out, npos),      # E' or P not whole pages
             (16, 32, bt, npos),                           # new table over the old one
             (16, 32, out, pos)]                           # new positions over the old
    for prefix, evict, o, np_ in cases:
        with pytest.raises(kv.KvError) as ei:
            kv.kv_compact_segment_remap(c, prefix, evict, o, pos, np_)
        assert ei.value.code == kv.KV_EINVAL
    with pytest.raises(ValueError):                                    # no block table
        kv.kv_compact_segment_remap(kv.PagedCache(k, v, 512), 16, 32, out, pos, npos)
    torch.cuda.synchronize()
    assert torch.equal(bt, bt0) and int(out.abs().sum()) == 0          # nothing was written


def _rows(t, table, idx):
    """Logical rows idx of a paged [layers][pages][16][heads][128] tensor, gathered on the
    device: [layers][len(idx)][heads][128]."""
    idx = np.asarray(idx, np.int64)
    pages = torch.from_numpy(table[idx // 16].astype(np.int64)).to(t.device)
    slots = torch.from_numpy(idx % 16).to(t.device)
    return t[:, pages, slots]


def _checksum(t):
    return int(t.view(torch.int16).sum(dtype=torch.int64))


def test_full_size_mistral_131k_segment_remap():
    """Mistral-7B shape at full size (32 layers, 131,072 tokens through a shuffled block
    table, 16,384-token prefix, 30% evicted): the remap with renumbering, every rank of
    the first and last layer against the oracle, V untouched, and sampled ranks of every
    layer."""
    w = synth.workload("mistral-7b-n131072-segment")
    N, NL = w.n_tokens, w.n_layers
    k, v, bt = synth.kv_cache(w, seed=0, device=DEV, paged_shuffle=True, extra_pages=4)
    n_keep, e = kv.kv_select_segment(N, w.segment_prefix, int(w.segment_frac * N), 16)
    keep = O.select_segment(N, w.segment_prefix, int(w.segment_frac * N), 16)
    assert len(keep) == n_keep
    layers = [0, NL - 1]
    btn = bt.cpu().numpy()
    edge_k = _rows(k[layers], btn, np.arange(N)).cpu()                 # bf16, converted per chunk
    edge_v = _rows(v[layers], btn, np.arange(N)).cpu()
    g = torch.Generator().manual_seed(5)
    ranks = sorted(set([0, w.segment_prefix - 1, w.segment_prefix, n_keep - 1]
                       + torch.randint(0, n_keep, (40,), generator=g).tolist()))
    srcs = keep[ranks]
    all_k = np64(_rows(k, btn, srcs))
    v_sum = _checksum(v)
    bt_out = torch.zeros(-(-n_keep // 16), dtype=torch.int32, device=DEV)
    new_pos = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
    kv.kv_compact_segment_remap(kv.PagedCache(k, v, N, bt), w.segment_prefix, e, bt_out,
                                torch.arange(N, dtype=torch.int32, device=DEV), new_pos, renumber_base=0,
                                rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    assert (new_pos.cpu().numpy() == np.arange(n_keep)).all()
    assert _checksum(v) == v_sum
    bto = bt_out.cpu().numpy()
    assert (bto == np.concatenate([btn[:w.segment_prefix // 16], btn[(w.segment_prefix + e) // 16:]])).all()
    gk = _rows(k[layers], bto, np.arange(n_keep)).cpu()
    gv = _rows(v[layers], bto, np.arange(n_keep)).cpu()
    step = 8192
    for r0 in range(0, n_keep, step):
        r1 = min(n_keep, r0 + step)
        src = torch.from_numpy(keep[r0:r1])
        rk, rv, _ = O.compact_rerope(np64(edge_k[:, src]), np64(edge_v[:, src]), np.arange(r1 - r0),
                                     keep[r0:r1], r0, w.rope_theta)
        assert (np64(gv[:, r0:r1]) == rv).all(), r0
        got = np64(gk[:, r0:r1])
        moved = keep[r0:r1] != np.arange(r0, r1)
        assert (got[:, ~moved] == rk[:, ~moved]).all(), r0
        assert_bf16_within_1ulp(got, rk, f"K ranks {r0}..{r1}")
    delta = np.array(ranks) - srcs
    rk = O.bf16_round(O.rope_rotate(all_k, delta[None, :, None], w.rope_theta))
    rk[:, delta == 0] = all_k[:, delta == 0]
    assert_bf16_within_1ulp(np64(_rows(k, bto, ranks)), rk, "K at N=131K, all layers")
    del k, v
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ page-list form

def _pages_case(nl, hkv, n, pg, budget_pages, base, theta, seed, pin_frac=0.05):
    """Page-mode selection on a paged row, then kv_compact_pages_remap; checked against the
    oracle read through the new table, the physical invariants and the gather form."""
    w = synth.workload("mistral-7b-n131072-segment", n_layers=nl, n_kv_heads=hkv, n_q_heads=4 * hkv, n_tokens=n,
                       page_size=pg)
    k, v, bt = synth.kv_cache(w, seed=seed, device=DEV, paged_shuffle=True, extra_pages=3)
    k0, v0 = k.clone(), v.clone()
    n_items = -(-n // pg)
    score = synth.scores(n_items, seed=seed, alphabet=[0.25, 0.5, 0.75] if seed % 2 else None)
    pinned = synth.pinned_mask(n_items, seed=seed, frac=pin_frac)
    max_keep = min(n, max(1, budget_pages) * pg + pg)
    keep = torch.full((max_keep,), -1, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_select(score.to(DEV), pinned.to(DEV), pg, n, budget_pages, keep, nk)
    g = torch.Generator().manual_seed(seed)
    old_pos = (torch.arange(n, dtype=torch.int32) + torch.randint(0, 30, (1,), generator=g).int()).to(DEV)
    out_pages = -(-max_keep // pg)
    bt_out = torch.full((out_pages,), -7, dtype=torch.int32, device=DEV)
    new_pos = torch.full((max_keep,), -7, dtype=torch.int32, device=DEV)
    span = torch.randint(-1, 100, (n,), generator=g, dtype=torch.int32).to(DEV)
    span_out = torch.full((max_keep,), -9, dtype=torch.int32, device=DEV)
    status = torch.full((1,), 0x55, dtype=torch.int32, device=DEV)
    kv.kv_compact_pages_remap(kv.PagedCache(k, v, n, bt), keep, nk, max_keep, bt_out, old_pos, new_pos,
                              renumber_base=base, rope_theta=theta, meta=[(span, span_out)], status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    items, _ = O.select_items(score.double().numpy(), pinned.numpy(), budget_pages)
    toks = O.expand_items(items, pg, n)
    n_keep = int(nk.item())
    assert n_keep == len(toks) and (keep.cpu().numpy()[:n_keep] == toks).all()
    btn, bto = bt.cpu().numpy(), bt_out.cpu().numpy()
    kp = -(-n_keep // pg)
    assert (bto[:kp] == btn[np.asarray(items, np.int64)]).all()
    op = old_pos.cpu().numpy()
    kl = unpage(np64(k0), btn, pg, n)
    vl = unpage(np64(v0), btn, pg, n)
    rk, rv, rpos = O.compact_rerope(kl, vl, toks, op, base, theta)
    assert (new_pos.cpu().numpy()[:n_keep] == rpos).all()
    assert (span_out.cpu().numpy()[:n_keep] == span.cpu().numpy()[toks]).all()
    gk = unpage(np64(k), bto[:kp], pg, n_keep)
    gv = unpage(np64(v), bto[:kp], pg, n_keep)
    assert (gv == rv).all()
    same = rpos == op[toks]
    assert (gk[:, same] == rk[:, same]).all()
    assert_bf16_within_1ulp(gk, rk, "relinked K")
    assert torch.equal(v, v0)
    # the gather form on the original row gives the same keys bit for bit
    dk = torch.zeros((nl, out_pages, pg, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    kv.kv_compact_rerope(kv.PagedCache(k0, v0, n, bt), kv.PagedCache(dk, dv, max_keep), keep, nk, max_keep,
                         old_pos, None, renumber_base=base, rope_theta=theta)
    torch.cuda.synchronize()
    assert (np64(dk).reshape(nl, -1, hkv, 128)[:, :n_keep] == gk).all()
    return n_keep


@pytest.mark.parametrize("nl,hkv,n,pg,budget_pages,base,theta,pin_frac", [
    (2, 8, 3000, 16, 40, 0, 1e4, 0.05),       # ragged last page (pinned pages include it sometimes)
    (2, 8, 3000, 16, 40, -1, 1e4, 0.05),      # positions kept: nothing but the table changes
    (3, 2, 2048, 64, 8, 5, 1e6, 0.05),        # large pages, renumbered from 5
    (1, 4, 777, 4, 50, 0, 1e6, 0.05),         # small pages
    (2, 2, 500, 16, 100, 0, 1e4, 0.05),       # budget above the row: every page kept
    (1, 1, 1_000_003, 16, 128, 0, 1e6, 5e-4),  # 62,501 pages (the last one partial) down to 128
])
def test_pages_remap_parity(nl, hkv, n, pg, budget_pages, base, theta, pin_frac):
    _pages_case(nl, hkv, n, pg, budget_pages, base, theta, seed=n + pg + budget_pages, pin_frac=pin_frac)


def test_pages_remap_refuses_to_move_partial_pages():
    """A keep list that is not whole pages: the entries that would leave their slots are
    left alone and the status reports it; values are never touched."""
    w = synth.workload("mistral-7b-n131072-segment", n_layers=1, n_kv_heads=2, n_q_heads=8, n_tokens=640)
    k, v, bt = synth.kv_cache(w, seed=3, device=DEV, paged_shuffle=True, extra_pages=2)
    k0, v0 = k.clone(), v.clone()
    toks = np.concatenate([np.arange(32, 48), np.arange(100, 110), np.arange(160, 176)]).astype(np.int32)
    keep = torch.from_numpy(toks).to(DEV)
    nk = torch.tensor([len(toks)], dtype=torch.int64, device=DEV)
    bt_out = torch.zeros(-(-len(toks) // 16), dtype=torch.int32, device=DEV)
    new_pos = torch.zeros(len(toks), dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kv_compact_pages_remap(kv.PagedCache(k, v, 640, bt), keep, nk, len(toks), bt_out,
                              torch.arange(640, dtype=torch.int32, device=DEV), new_pos, renumber_base=-1,
                              status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kv.KV_STATUS_NOT_WHOLE_PAGES
    assert torch.equal(v, v0) and torch.equal(k, k0)
    # the whole first page was relinked and its positions written
    assert (new_pos.cpu().numpy()[:16] == np.arange(32, 48)).all()
