"""Seeded sweeps over shapes the fixed parity cases do not name.

Every configuration is drawn from a fixed seed, so a failure names its case and replays
exactly.  Each one is held to the bars of the parity tests: selection bit-exact against
the oracle (keep list, count and status word), compaction with V and unrotated K
bit-exact and rotated K within 1 bf16 ulp, attention mass and scores within 1e-5
relative, LSE within 1e-5 absolute."""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
import synth
import test_gpu_parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _select_cases(n_cases=100, seed=2024):
    rng = np.random.default_rng(seed)
    sizes = [1, 2, 3, 17, 63, 64, 65, 1000, 4095, 4096, 4097, 8191, 12_288, 50_000, 130_000]
    for c in range(n_cases):
        n_items = int(rng.choice(sizes)) + (int(rng.integers(0, 50)) if rng.random() < 0.3 else 0)
        it = int(rng.choice([1, 1, 16, 64]))
        n_tokens = n_items * it - (int(rng.integers(0, it)) if it > 1 else 0)
        alphabet = None if rng.random() < 0.6 else [float(x) for x in rng.choice([-1.0, 0.0, 0.5, 1.0, 2.0], 3)]
        nan = float(rng.choice([0.0, 0.0, 0.01]))
        negz = bool(rng.random() < 0.3)
        pin = float(rng.choice([0.0, 0.01, 0.3]))
        budget = int(rng.integers(0, n_items + 4))
        cap = None if rng.random() < 0.7 else int(rng.integers(1, max(2, budget * it + 1)))
        yield c, n_items, it, n_tokens, alphabet, nan, negz, pin, budget, cap


@pytest.mark.parametrize("case", list(_select_cases()), ids=lambda c: f"sel{c[0]}")
def test_select_sweep(case):
    c, n_items, it, n_tokens, alphabet, nan, negz, pin, budget, cap = case
    print(f"select sweep {c}: items={n_items} it={it} tokens={n_tokens} budget={budget} cap={cap}", flush=True)
    s = synth.scores(n_items, seed=100 + c, alphabet=alphabet, nan_frac=nan, neg_zero=negz)
    p = synth.pinned_mask(n_items, seed=100 + c, frac=pin) if pin else None
    P._select_case(n_items, it, n_tokens, budget, s, p, cap=cap)


def _compact_cases(n_cases=40, seed=77):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        nl = int(rng.integers(1, 5))
        hkv = int(rng.choice([1, 2, 4, 8]))
        src_ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        dst_ps = int(rng.choice([1, 4, 16, 128]))
        n = int(rng.integers(1, 3000))
        n_keep = int(rng.integers(1, n + 1))
        base = int(rng.choice([-1, 0, int(rng.integers(1, 5000))]))
        theta = float(rng.choice([1e4, 1e6, 5e5]))
        yield c, nl, hkv, src_ps, dst_ps, n, n_keep, base, theta, bool(rng.random() < 0.5)


@pytest.mark.parametrize("case", list(_compact_cases()), ids=lambda c: f"cmp{c[0]}")
def test_compact_sweep(case):
    c, nl, hkv, src_ps, dst_ps, n, n_keep, base, theta, shuffle = case
    print(f"compact sweep {c}: layers={nl} kv_heads={hkv} pages {src_ps}->{dst_ps} n={n} keep={n_keep} "
          f"base={base}", flush=True)
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n,
                       page_size=src_ps)
    k, v, bt = synth.kv_cache(w, seed=500 + c, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    g = torch.Generator().manual_seed(600 + c)
    keep = torch.sort(torch.randperm(n, generator=g)[:n_keep])[0].to(torch.int32)
    old_pos = torch.arange(n, dtype=torch.int32) + torch.randint(0, 200_000, (n,), generator=g, dtype=torch.int32)
    n_dst_pages = -(-n_keep // dst_ps) + 1
    dk = torch.zeros((nl, n_dst_pages, dst_ps, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    dbt = torch.randperm(n_dst_pages, generator=g)[: -(-n_keep // dst_ps)].to(torch.int32).to(DEV) \
        if shuffle else None
    meta_src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), generator=g, dtype=torch.int32)
    meta_dst = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
    new_pos = torch.full((n_keep,), -7, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, n, bt), kv.PagedCache(dk, dv, n_keep, dbt), keep.to(DEV), None,
                         n_keep, old_pos.to(DEV), new_pos, renumber_base=base, rope_theta=theta, limit=0,
                         meta=[(meta_src.to(DEV), meta_dst)])
    torch.cuda.synchronize()
    kl = P._paged_to_logical(k, bt, src_ps, n)
    vl = P._paged_to_logical(v, bt, src_ps, n)
    rk, rv, rpos = O.compact_rerope(kl, vl, keep.numpy(), old_pos.numpy(), base, theta)
    gk = P._paged_to_logical(dk, dbt, dst_ps, n_keep)
    gv = P._paged_to_logical(dv, dbt, dst_ps, n_keep)
    assert (new_pos.cpu().numpy() == rpos).all()
    assert (gv == rv).all()
    still = rpos == old_pos.numpy()[keep.numpy()]
    assert (gk[:, still] == rk[:, still]).all()
    P.assert_bf16_within_1ulp(gk, rk, f"compact sweep {c}")
    assert (meta_dst.cpu() == meta_src[keep.long()]).all()


def _score_cases(n_cases=40, seed=5):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
        w_ = int(rng.integers(1, 65))
        while g * w_ > 512 or (1 << max(0, (g - 1).bit_length())) * w_ > 512:
            w_ //= 2
        n = int(rng.integers(max(w_, 2), 5000))
        yield (c, hkv, g, max(w_, 1), n, int(rng.integers(1, 3)), int(rng.choice([1, 4, 16, 64])),
               str(rng.choice(["sum", "max_group"])), bool(rng.random() < 0.5))


@pytest.mark.parametrize("case", list(_score_cases()), ids=lambda c: f"score{c[0]}")
def test_score_sweep(case):
    c, hkv, g, win, n, nl, ps, agg, spans = case
    print(f"score sweep {c}: kv_heads={hkv} G={g} W={win} N={n} layers={nl} page={ps} {agg} spans={spans}",
          flush=True)
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=n, window=win, n_q_heads=hkv * g, n_kv_heads=hkv,
                       n_layers=nl, page_size=ps, n_spans=30)
    k, v, bt = synth.kv_cache(w, seed=700 + c, device="cpu", paged_shuffle=True, extra_pages=2)
    q = synth.window_queries(w, seed=700 + c)
    kw = dict(n_sink=min(4, n), n_recent=min(16, n))
    ref_kw = dict(kw)
    if spans:
        sid, sb = synth.spans(w, seed=700 + c, p_needed=0.3)
        kw.update(span_id=sid.to(DEV), span_bonus=sb.to(DEV))
        ref_kw.update(span_id=sid.numpy(), span_bonus=sb.numpy())
    acc0 = synth.h2o_state(w, seed=700 + c)
    acc = acc0.to(DEV)
    got = P._run_score(w, k.to(DEV), v.to(DEV), bt.to(DEV), q, policy="h2o", item_tokens=1,
                       state=dict(accum=acc), aggregate=agg, **kw)
    kl = O.gather_logical(P.np64(k), bt.numpy(), ps, n)
    ref = O.score_step(P.np64(q), kl, policy="h2o", accum=P.np64(acc0), aggregate=agg, **ref_kw)
    P.assert_rel(P.np64(got["mass"]), ref["mass"], what=f"score sweep {c} mass")
    assert np.abs(P.np64(got["lse"]) - ref["lse"]).max() < 1e-5
    P.assert_rel(P.np64(acc.cpu()), ref["accum"], what="accum")
    P.assert_rel(P.np64(got["item_score"]), ref["item_score"], what="score")
    assert (got["item_pinned"].numpy().astype(bool) == ref["item_pinned"]).all()


@pytest.mark.parametrize("case", list(_score_cases(n_cases=20, seed=6)), ids=lambda c: f"memdecay{c[0]}")
def test_memdecay_sweep(case):
    """MemDecay over the same kind of shapes, tokens or pages as items (the sum over query
    heads, as MemDecay defines the mass), with region pins, sinks, recent tokens and spans."""
    c, hkv, g, win, n, nl, ps, _, spans = case
    pages = bool(c % 2)
    print(f"memdecay sweep {c}: kv_heads={hkv} G={g} W={win} N={n} layers={nl} page={ps} page_items={pages}",
          flush=True)
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=n, window=win, n_q_heads=hkv * g, n_kv_heads=hkv,
                       n_layers=nl, page_size=ps, n_spans=30, system_prefix=min(32, n))
    k, v, bt, q = P._make_score_inputs(w, seed=800 + c, shuffle=True)
    st0 = P._memdecay_state(w, seed=800 + c)
    dev = {key: t.clone().to(DEV) for key, t in st0.items()}
    kw, sid, sb = {}, None, None
    if spans:
        sid, sb = synth.spans(w, seed=800 + c, p_needed=0.3)
        kw = dict(span_id=sid.to(DEV), span_bonus=sb.to(DEV))
    item_tokens = ps if pages else 1
    n_sink, n_recent = min(4, n), min(16, n)
    got = P._run_score(w, k, v, bt, q, policy="memdecay", item_tokens=item_tokens, state=dev, rho=w.rho,
                       alpha=w.alpha, tau=w.tau, dt_steps=2, pinned_regions=0b101, n_sink=n_sink,
                       n_recent=n_recent, **kw)
    dev_state = {key: t.cpu() for key, t in dev.items()}
    kl = P._paged_to_logical(k, bt, ps, n)
    P._compare_memdecay(w, q, kl, st0, dev_state, got, w.rho, w.alpha, w.tau, 2, item_tokens, 0b101,
                        n_sink=n_sink, n_recent=n_recent, span_id=sid, span_bonus=sb)


def _lrfu_cases(n_cases=30, seed=11):
    rng = np.random.default_rng(seed)
    dists = ["power", "ties", "mixed", "equal", "tiny", "wide", "twobinade"]
    for c in range(n_cases):
        n = int(rng.choice([1, 2, 5, 63, 64, 65, 1000, 4096, 4097, 30_000, 100_000, 250_000]))
        dist = str(rng.choice(dists))
        p = float(np.float32(rng.choice([0.0, 1.0, rng.random(), rng.random(), 0.9, 0.5])))
        scale = float(rng.choice([1.0, 1.0 / (36 * 8 * 64), 1e-20, 3.0]))
        decay = float(rng.choice([0.0, 0.5, 1.0, rng.random()]))
        yield c, n, dist, p, scale, decay


@pytest.mark.parametrize("case", list(_lrfu_cases()), ids=lambda c: f"lrfu{c[0]}")
def test_lrfu_sweep(case):
    import test_gpu_actkv as A
    c, n, dist, p, scale, decay = case
    print(f"lrfu sweep {c}: n={n} {dist} p={p!r} scale={scale} decay={decay}", flush=True)
    rng = np.random.default_rng(900 + c)
    a = A._scores(rng, n, dist)
    ks0 = (rng.random(n) * 2).astype(np.float32)
    s = (a * np.float32(scale)).astype(np.float32)
    ks_ref, hit_ref = O.lrfu_update(ks0.astype(np.float64), s, p=p, decay=np.float32(decay))
    ks = torch.from_numpy(ks0).to(DEV)
    hit = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
    kv.kv_lrfu_update(torch.from_numpy(a).to(DEV), ks, scale=scale, top_p=p, decay=decay, hit=hit)
    torch.cuda.synchronize()
    got_hit = hit.cpu().numpy().astype(bool)
    assert (got_hit == hit_ref).all(), (int((got_hit != hit_ref).sum()), int(hit_ref.sum()))
    np.testing.assert_allclose(ks.cpu().numpy().astype(np.float64), ks_ref, rtol=1e-6, atol=1e-37)


def _tail_cases(n_cases=20, seed=12):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        n = int(rng.integers(1, 4000))
        budget = int(rng.integers(1, n + 20))
        n_keep = int(rng.integers(0, min(n, budget) + 1))
        yield c, n, budget, n_keep, bool(rng.random() < 0.5), int(rng.integers(1, 4)), int(rng.choice([1, 2, 8]))


@pytest.mark.parametrize("case", list(_tail_cases()), ids=lambda c: f"tail{c[0]}")
def test_tail_compact_sweep(case):
    import test_gpu_actkv as A
    c, n, budget, n_keep, shuffle, nl, hkv = case
    print(f"tail sweep {c}: n={n} budget={budget} keep={n_keep} layers={nl} kv_heads={hkv}", flush=True)
    rng = np.random.default_rng(1000 + c)
    slots = -(-n // 16) * 16
    k = O.bf16_round(rng.standard_normal((nl, slots, hkv, 128)))
    v = O.bf16_round(rng.standard_normal((nl, slots, hkv, 128)))
    pos = rng.integers(0, 2 ** 31 - 1, slots).astype(np.int32)
    keep = np.sort(rng.choice(n, n_keep, replace=False)) if n_keep else np.zeros(0, np.int64)
    kt, bt = A._paged(rng, k, shuffle)
    vt = torch.zeros_like(kt)
    vt_l, _ = A._paged(np.random.default_rng(0), v, False)
    for pg in range(slots // 16):
        vt[:, int(bt[pg]) if bt is not None else pg] = vt_l[:, pg]
    pos_d = torch.from_numpy(pos).to(DEV)
    keep_d = torch.from_numpy(np.concatenate([keep, [0]]).astype(np.int32)).to(DEV)
    status = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    start = kv.kv_compact_tail_inplace(kv.PagedCache(kt, vt, n, bt), keep_d, None, len(keep), budget,
                                       meta=[pos_d], status=status)
    torch.cuda.synchronize()
    if budget >= n:
        assert start == 0
        src = dst = np.zeros(0, dtype=np.int64)
    else:
        s0, _, src, dst, over = O.tail_compaction_pairs(n, keep, budget, 16)
        assert start == s0 and not over
    assert int(status.item()) == 0
    assert (A._logical(kt, bt, slots) == O.tail_compact(k, src, dst)).all()
    assert (A._logical(vt, bt, slots) == O.tail_compact(v, src, dst)).all()
    assert (pos_d.cpu().numpy() == O.tail_compact(pos[None], src, dst)[0]).all()


def _swap_cases(n_cases=12, seed=13):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        count = int(rng.integers(1, 2500))
        chunk = int(rng.choice([1, 7, 64, 256, 1024, 4096]))
        buf = min(chunk, count)
        if rng.random() < 0.5:                 # buffer before the incoming rows
            buf_first = int(rng.integers(0, 50))
            in_first = buf_first + buf + int(rng.integers(0, 50))
        else:
            in_first = int(rng.integers(0, 50))
            buf_first = in_first + count + int(rng.integers(0, 50))
        yield c, count, chunk, in_first, buf_first, bool(rng.random() < 0.5), bool(rng.random() < 0.5)


@pytest.mark.parametrize("case", list(_swap_cases()), ids=lambda c: f"swap{c[0]}")
def test_swap_sweep(case):
    """Penelope's both-tiers-full swap against the oracle's chunk-by-chunk swap."""
    import test_gpu_offload as F
    c, count, chunk, in_first, buf_first, shuffle, two_streams = case
    print(f"swap sweep {c}: count={count} chunk={chunk} in_first={in_first} buf_first={buf_first} "
          f"two_streams={two_streams}", flush=True)
    nl, hkv, n = 2, 2, 3000
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=1100 + c, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    k0, v0 = F._logical(k, bt, n), F._logical(v, bt, n)
    rng = np.random.default_rng(1200 + c)
    rows = max(in_first + count, buf_first + min(chunk, count)) + 5
    pk = O.bf16_round(rng.standard_normal((nl, rows, hkv, 128)))
    pv = O.bf16_round(rng.standard_normal((nl, rows, hkv, 128)))
    hk = torch.from_numpy(pk).to(torch.bfloat16).pin_memory()
    hv = torch.from_numpy(pv).to(torch.bfloat16).pin_memory()
    slots = rng.choice(n, min(count, n), replace=False)
    count = len(slots)
    in_stream = torch.cuda.Stream() if two_streams else None
    slots_d = torch.from_numpy(slots.astype(np.int32)).to(DEV)
    torch.cuda.synchronize()
    out_rows, nxt, _ = kv.kv_swap_chunked(kv.PagedCache(k, v, n, bt), slots_d, hk, hv, in_first, buf_first,
                                          chunk=chunk, in_stream=in_stream)
    torch.cuda.current_stream().synchronize()
    gk, pk2, want_rows, want_next = O.chunked_swap(k0, pk, slots, in_first, buf_first, chunk)
    gv, pv2, _, _ = O.chunked_swap(v0, pv, slots, in_first, buf_first, chunk)
    assert out_rows == want_rows.tolist() and nxt == want_next
    assert (F._logical(k, bt, n) == gk).all() and (F._logical(v, bt, n) == gv).all()
    assert (hk.double().numpy() == pk2).all() and (hv.double().numpy() == pv2).all()


def _store_cases(n_cases=8, seed=14):
    rng = np.random.default_rng(seed)
    kinds = [("default", {}), ("linear", dict(factor=4.0)),
             ("llama3", dict(factor=8.0, original_max_position=8192)),
             ("yarn", dict(factor=16.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0))]
    for c in range(n_cases):
        kind, kw = kinds[int(rng.integers(0, len(kinds)))]
        yield (c, int(rng.integers(1, 4)), int(rng.choice([1, 2, 8])), int(rng.integers(100, 1500)), kind, kw,
               float(rng.uniform(0.3, 0.95)), bool(rng.random() < 0.5))


@pytest.mark.parametrize("case", list(_store_cases()), ids=lambda c: f"store{c[0]}")
def test_reference_store_sweep(case):
    """Three compaction steps through PACE's reference store (renumbering, new tokens
    between steps, sometimes a stale entry), each GPU step from the oracle's state."""
    import test_gpu_store as S
    c, nl, hkv, n0, kind, kw, frac, plant = case
    print(f"store sweep {c}: layers={nl} kv_heads={hkv} n={n0} {kind} keep={frac:.2f} stale={plant}", flush=True)
    rng = np.random.default_rng(1300 + c)
    inv = O.scaled_inv_freq(kind, 5e5, **kw)
    rope = kv.kv_rope(kind, base=5e5, **kw)
    k, v, pos, ref_k, ref_pos = S._state(rng, nl, n0, hkv)
    for step in range(3):
        n = k.shape[1]
        if plant and step == 2 and (ref_pos != O.REF_NONE).any():
            j = int(np.nonzero(ref_pos != O.REF_NONE)[0][-1])
            ref_k[:, j] = O.bf16_round(rng.standard_normal((nl, hkv, 128)))
        n_keep = max(1, int(n * frac))
        keep = np.sort(rng.choice(n, n_keep, replace=False))
        base = int(rng.integers(0, 100))
        ok, ov, opos, oref, orefp, _ = O.compact_rerope_store(k, v, keep, pos, base, inv, ref_k, ref_pos)
        kt, bt = S.to_paged(k, rng)
        vt = torch.zeros_like(kt)
        vl = torch.from_numpy(v).to(torch.bfloat16).to(DEV)
        for p in range(-(-n // S.PG)):
            seg = vl[:, p * S.PG:(p + 1) * S.PG]
            vt[:, int(bt[p]), : seg.shape[1]] = seg
        src_store = S.store_to_dev(ref_k, ref_pos)
        dst_store = kv.RefStore.empty(nl, n_keep, hkv, DEV)
        dk = torch.zeros((nl, -(-n_keep // S.PG), S.PG, hkv, 128), dtype=torch.bfloat16, device=DEV)
        dv = torch.zeros_like(dk)
        newp = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
        kv.kv_compact_rerope(kv.PagedCache(kt, vt, n, bt), kv.PagedCache(dk, dv, n_keep),
                             torch.from_numpy(keep.astype(np.int32)).to(DEV), None, n_keep,
                             torch.from_numpy(pos.astype(np.int32)).to(DEV), newp, renumber_base=base,
                             rope=rope, ref_src=src_store, ref_dst=dst_store)
        torch.cuda.synchronize()
        gp = dst_store.pos.cpu().numpy().astype(np.int64)
        assert (newp.cpu().numpy() == opos).all(), step
        assert (S.from_paged(dv, None, n_keep) == ov).all(), step
        assert (gp == orefp).all(), step
        valid = orefp != O.REF_NONE
        gref = dst_store.k.float().cpu().double().numpy()
        assert (gref[:, valid] == oref[:, valid]).all(), step
        assert S.within_1ulp(S.from_paged(dk, None, n_keep), ok), step
        add = int(rng.integers(1, 200))
        k_new, v_new, _, _, _ = S._state(rng, nl, add, hkv)
        k = np.concatenate([ok, k_new], axis=1)
        v = np.concatenate([ov, v_new], axis=1)
        pos = np.concatenate([opos, opos.max() + 1 + np.arange(add)])
        ref_k = np.concatenate([oref, np.zeros_like(k_new)], axis=1)
        ref_pos = np.concatenate([orefp, np.full(add, O.REF_NONE, dtype=np.int64)])


def _remap_cases(n_cases=30, seed=515):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        pg = int(rng.choice([1, 2, 4, 8, 16, 64]))
        nl = int(rng.integers(1, 4))
        hkv = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 3000))
        pages = -(-n // pg)
        pp = int(rng.integers(0, pages + 1))
        full = n // pg                         # evicted pages must lie inside the row
        ep = int(rng.integers(0, max(1, full - pp + 1))) if full > pp else 0
        base = int(rng.choice([-1, 0, int(rng.integers(1, 4000))]))
        theta = float(rng.choice([1e4, 1e6]))
        yield c, nl, hkv, n, pg, pp * pg, ep * pg, base, theta


@pytest.mark.parametrize("case", list(_remap_cases()), ids=lambda c: f"remap{c[0]}")
def test_segment_remap_sweep(case):
    import test_gpu_remap as R
    c, nl, hkv, n, pg, prefix, evict, base, theta = case
    if prefix + evict > n:
        prefix = (n - evict) // pg * pg
    print(f"remap sweep {c}: layers={nl} kv_heads={hkv} tokens={n} page={pg} prefix={prefix} evict={evict} "
          f"base={base}", flush=True)
    R._case(nl, hkv, n, prefix, evict, base, theta, seed=900 + c, pg=pg)


def _pages_remap_cases(n_cases=20, seed=616):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        pg = int(rng.choice([1, 2, 4, 8, 16, 64]))
        nl = int(rng.integers(1, 4))
        hkv = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 2500))
        pages = -(-n // pg)
        budget = int(rng.integers(0, pages + 3))
        base = int(rng.choice([-1, 0, int(rng.integers(1, 4000))]))
        theta = float(rng.choice([1e4, 1e6]))
        yield c, nl, hkv, n, pg, budget, base, theta


@pytest.mark.parametrize("case", list(_pages_remap_cases()), ids=lambda c: f"pages{c[0]}")
def test_pages_remap_sweep(case):
    import test_gpu_remap as R
    c, nl, hkv, n, pg, budget, base, theta = case
    print(f"pages remap sweep {c}: layers={nl} kv_heads={hkv} tokens={n} page={pg} budget={budget} base={base}",
          flush=True)
    R._pages_case(nl, hkv, n, pg, budget, base, theta, seed=700 + c, pin_frac=0.0)
