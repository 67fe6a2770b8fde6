"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bars (stated once here and used below):
  * kept indices, compacted V, unrotated K, positions, metadata: bit-exact;
  * re-rotated bf16 keys: within 1 bf16 ulp of the oracle's correctly rounded value;
  * attention mass, token/page scores, EWMA: within 1e-5 relative (fp32 vs fp64);
    LSE within 1e-5 absolute (it is a logarithm);
  * decay clocks: exact, except tokens whose windowed mass lies within 1e-5 relative of
    tau, where an fp32-vs-fp64 difference may legitimately flip the reset;
  * end to end (each side scores for itself): kept sets may differ only in items whose
    oracle score is within 1e-5 relative of the selection threshold.
"""
import math

import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
from layout import unpage
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-5


def np64(t):
    return t.detach().cpu().double().numpy() if t.dtype != torch.bfloat16 else \
        t.detach().float().cpu().double().numpy()


def f32(x):
    """Round a Python/NumPy value to float32 (what the device receives)."""
    return np.float32(x).astype(np.float64)


def assert_rel(got, ref, rtol=RTOL, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bad = np.abs(got - ref) > rtol * np.abs(ref) + 1e-35
    assert not bad.any(), (what, int(bad.sum()), got[bad][:5], ref[bad][:5])


def ulp_bf16(x):
    """Spacing of bf16 values at |x|: 2**(e-8) for |x| in [2**(e-1), 2**e), never below the
    subnormal spacing 2**-133 (which is also the spacing at 0)."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(x)
    return np.where(x == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def assert_bf16_within_1ulp(got, ref, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bad = np.abs(got - ref) > ulp_bf16(ref)
    assert not bad.any(), (what, int(bad.sum()), got[bad][:5], ref[bad][:5])


# ------------------------------------------------------------------------------ compaction

def _paged_to_logical(t, bt, pg, n):
    return unpage(np64(t), None if bt is None else bt.cpu().numpy(), pg, n)


@pytest.mark.parametrize("nl,hkv,n,n_keep,shuffle,base,theta", [
    (1, 2, 512, 128, False, 0, 1e6),
    (3, 2, 1000, 333, True, 0, 1e6),
    (2, 8, 777, 100, True, -1, 1e4),
    (2, 8, 4096, 1, False, 5, 1e4),
    (28, 2, 2048, 512, True, 0, 1e6),
    (5, 8, 600, 150, True, 3, 1e6),     # 320 items per token: two workgroups of 160
])
def test_compact_rerope_parity(nl, hkv, n, n_keep, shuffle, base, theta):
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=n, device=DEV, paged_shuffle=shuffle, extra_pages=3)
    g = torch.Generator().manual_seed(n + 1)
    keep = torch.sort(torch.randperm(n, generator=g)[:n_keep])[0].to(torch.int32)
    # old positions: some tokens were renumbered before (delta 0 for some, up to ~1e6)
    old_pos = torch.arange(n, dtype=torch.int32) + torch.randint(0, 1_000_000, (n,), generator=g,
                                                                   dtype=torch.int32)
    old_pos[keep[: max(1, n_keep // 4)]] = torch.arange(max(1, n_keep // 4), dtype=torch.int32) + max(base, 0)
    region = torch.randint(0, 7, (n,), generator=g, dtype=torch.int32).to(torch.uint8)
    ewma = torch.rand(n, generator=g)
    span = torch.randint(-1, 200, (n,), generator=g, dtype=torch.int32)
    big = torch.randint(-2 ** 62, 2 ** 62, (n,), generator=g, dtype=torch.int64)
    n_dst_pages = -(-n_keep // 16) + 2
    dk = torch.zeros((nl, n_dst_pages, 16, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    dbt = torch.randperm(n_dst_pages, generator=g)[: -(-n_keep // 16)].to(torch.int32).to(DEV) if shuffle else None
    src = kv.PagedCache(k, v, n, bt)
    dst = kv.PagedCache(dk, dv, n_keep, dbt)
    outs = [torch.zeros(n_keep, dtype=x.dtype, device=DEV) for x in (region, ewma, span, big)]
    new_pos = torch.full((n_keep,), -7, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(src, dst, keep.to(DEV), None, n_keep, old_pos.to(DEV), new_pos,
                         renumber_base=base, rope_theta=theta, limit=0,
                         meta=[(x.to(DEV), o) for x, o in zip((region, ewma, span, big), outs)])
    torch.cuda.synchronize()
    kl = _paged_to_logical(k, bt, 16, n)
    vl = _paged_to_logical(v, bt, 16, n)
    rk, rv, rpos = O.compact_rerope(kl, vl, keep.numpy(), old_pos.numpy(), base, theta)
    gk = _paged_to_logical(dk, dbt, 16, n_keep)
    gv = _paged_to_logical(dv, dbt, 16, n_keep)
    assert (new_pos.cpu().numpy() == rpos).all()
    assert (gv == rv).all(), "V must be bit-exact"
    delta = rpos - old_pos.numpy()[keep.numpy()]
    still = delta == 0
    assert (gk[:, still] == rk[:, still]).all(), "unrotated K must be bit-exact"
    assert_bf16_within_1ulp(gk[:, ~still], rk[:, ~still], "rotated K")
    exact = (gk[:, ~still] == rk[:, ~still]).mean() if (~still).any() else 1.0
    assert exact > 0.999
    for x, o in zip((region, ewma, span, big), outs):
        assert (o.cpu() == x[keep.long()]).all()


def test_compact_respects_device_count():
    w = synth.workload("qwen2.5-1.5b-1layer-n512")
    k, v, _ = synth.kv_cache(w, seed=1, device=DEV)
    keep = torch.arange(0, 512, 4, dtype=torch.int32, device=DEV)
    n_keep = torch.tensor([50], dtype=torch.int64, device=DEV)
    dk = torch.zeros((1, 8, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    pos = torch.arange(512, dtype=torch.int32, device=DEV)
    newp = torch.full((128,), -1, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, 512), kv.PagedCache(dk, dv, 128), keep, n_keep, 128, pos,
                         newp, renumber_base=0, rope_theta=1e6)
    torch.cuda.synchronize()
    flat = dk.reshape(1, 128, 2, 128)
    assert (flat[:, 50:] == 0).all() and (newp[50:] == -1).all() and (newp[:50] == torch.arange(50, device=DEV)).all()
    assert (flat[:, 1:50] != 0).any()


@pytest.mark.parametrize("nl,n,prefix,frac,base,theta,shuffle", [
    (2, 1000, 100, 0.3, 0, 1e4, False),
    (3, 4096, 512, 0.3, 0, 1e4, True),
    (2, 600, 0, 0.9, -1, 1e4, False),
    (2, 300, 200, 0.05, 7, 1e6, False),
    (9, 2000, 64, 0.3, 5, 1e6, True),  # 576 items per token: three workgroups; prefix shifted
])
def test_segment_inplace_parity(nl, n, prefix, frac, base, theta, shuffle):
    w = synth.workload("mistral-7b-n131072-segment", n_layers=nl, n_tokens=n)
    k, v, bt = synth.kv_cache(w, seed=n, device=DEV, paged_shuffle=shuffle, extra_pages=2)
    n_keep, e = kv.kv_select_segment(n, prefix, int(frac * n), 16)
    keep = O.select_segment(n, prefix, int(frac * n), 16)
    assert n_keep == len(keep)
    kl = _paged_to_logical(k, bt, 16, n)
    vl = _paged_to_logical(v, bt, 16, n)
    pos = torch.arange(n, dtype=torch.int32, device=DEV)
    region = torch.randint(0, 7, (n,), dtype=torch.int32).to(torch.uint8)
    reg_dev = region.to(DEV)
    kv.kv_compact_segment_inplace(kv.PagedCache(k, v, n, bt), prefix, e, pos, renumber_base=base,
                                  rope_theta=theta, meta=[reg_dev])
    torch.cuda.synchronize()
    rk, rv, rpos = O.compact_rerope(kl, vl, keep, np.arange(n), base, theta)
    gk = _paged_to_logical(k, bt, 16, n)[:, :n_keep]
    gv = _paged_to_logical(v, bt, 16, n)[:, :n_keep]
    assert (pos[:n_keep].cpu().numpy() == rpos).all()
    assert (gv == rv).all()
    delta = rpos - keep
    assert (gk[:, delta == 0] == rk[:, delta == 0]).all()
    assert_bf16_within_1ulp(gk, rk, "segment K")
    assert (reg_dev[:n_keep].cpu().numpy() == region.numpy()[keep]).all()


# ------------------------------------------------------------------------------ selection

def _select_case(n_items, item_tokens, n_tokens, budget, score, pinned, cap=None):
    cap = cap if cap is not None else n_tokens
    keep = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=DEV)
    n_keep = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kv_select(score.to(DEV), None if pinned is None else pinned.to(DEV), item_tokens, n_tokens, budget,
                 keep[:cap] if cap else keep[:1], n_keep, status)
    torch.cuda.synchronize()
    items, st = O.select_items(score.double().numpy(), None if pinned is None else pinned.numpy(), budget)
    toks = O.expand_items(items, item_tokens, n_tokens)
    nk = int(n_keep.item())
    assert nk == len(toks), (nk, len(toks))
    assert (keep[: min(nk, cap)].cpu().numpy() == toks[:cap]).all()
    want = st | (kv.KV_STATUS_KEEP_OVERFLOW if len(toks) > cap else 0)
    assert int(status.item()) == want


@pytest.mark.parametrize("n,alphabet,pin_frac,budget_frac,nan,negz", [
    (1, None, 0.0, 1.0, 0, False),
    (5, [0.0, 0.5, 1.0], 0.2, 0.6, 0, True),
    (100, [0.1, 0.2], 0.1, 0.3, 0, False),
    # rows of at most 4,096 items take the one-block kernel: the largest such row with
    # NaN, -0 and pins, ties at T, pinned items over the budget, every item kept
    (4096, None, 0.02, 0.1, 0.01, True),
    (4096, [0.0, 1.0], 0.01, 0.5, 0, True),
    (3000, None, 0.5, 0.1, 0.002, False),
    (2500, [0.5, 0.25], 0.1, 1.0, 0, False),
    (4097, None, 0.02, 0.1, 0.01, True),
    (100_000, None, 0.0013, 0.02048, 0, False),
    (100_000, [1.0, 2.0, 3.0], 0.05, 0.5, 0, False),
    (300_000, None, 0.3, 0.2, 0.001, True),        # pinned exceed the budget
    (62_500, None, 0.0, 0.002048, 0, False),
    # more than 4,096 items per block: several load batches per block, a ragged last one
    (1_000_000, None, 0.000132, 0.002048, 0.0001, True),
    (600_001, [1.0, 2.0, 3.0], 0.01, 0.3, 0, False),   # ties at T spread over many blocks
])
def test_select_token_mode(n, alphabet, pin_frac, budget_frac, nan, negz):
    s = synth.scores(n, seed=n, alphabet=alphabet, nan_frac=nan, neg_zero=negz)
    pin = synth.pinned_mask(n, seed=n, frac=pin_frac) if pin_frac else None
    _select_case(n, 1, n, int(round(budget_frac * n)), s, pin)


@pytest.mark.parametrize("n_tokens,budget_pages", [(512, 8), (2048, 32), (1000, 20), (1_000_000, 128),
                                                   (17, 2), (16, 0)])
def test_select_page_mode(n_tokens, budget_pages):
    n_items = -(-n_tokens // 16)
    s = synth.scores(n_items, seed=n_tokens, alphabet=[0.25, 0.5, 0.75] if n_tokens < 5000 else None)
    pin = synth.pinned_mask(n_items, seed=n_tokens, frac=0.05)
    _select_case(n_items, 16, n_tokens, budget_pages, s, pin)


def test_select_nan_only_in_pinned_items():
    """KV_STATUS_NAN_SCORE reports a NaN score of any item, also when only pinned items
    have one (they are kept whatever their score)."""
    s = synth.scores(5000, seed=12)
    pin = torch.zeros(5000, dtype=torch.uint8)
    pin[[7, 4000]] = 1
    s[[7, 4000]] = float("nan")
    _select_case(5000, 1, 5000, 300, s, pin)
    s2 = synth.scores(50, seed=13)
    p2 = torch.zeros(50, dtype=torch.uint8)
    p2[49] = 1
    s2[49] = float("nan")
    _select_case(50, 1, 50, 0, s2, p2)                 # pinned over budget as well


def test_select_short_rows_every_class():
    """Rows of 1 to 300 items (the one-block kernel ranks rows of at most 256 by counting,
    longer ones by histogram passes): scores drawn from a small set with ties, NaN, +-0 and
    +-inf, pins, budgets from 0 to past the row, token and page items (partial last
    pages), small keep capacities; each against the oracle's selection."""
    rng = np.random.default_rng(256)
    palette = np.array([np.nan, -np.inf, -1.5, -0.0, 0.0, 0.25, 0.5, 0.5, 1.0, np.inf], np.float32)
    for case in range(160):
        n_items = int(rng.integers(1, 301)) if case % 4 else int(rng.choice([1, 2, 255, 256, 257, 300]))
        if case % 3 == 0:
            s = rng.choice(palette, n_items).astype(np.float32)
        else:
            s = rng.random(n_items).astype(np.float32)
            s[rng.random(n_items) < 0.2] = s[0]                      # exact ties
        pin = (rng.random(n_items) < rng.choice([0.0, 0.05, 0.5])).astype(np.uint8)
        it = int(rng.choice([1, 1, 16]))
        n_tokens = n_items * it - (int(rng.integers(0, it)) if it > 1 else 0)
        budget = int(rng.integers(0, n_items + 6))
        cap = None if case % 5 else max(1, int(rng.integers(1, n_tokens + 1)))
        _select_case(n_items, it, n_tokens, budget, torch.from_numpy(s),
                     torch.from_numpy(pin) if pin.any() or case % 2 else None, cap=cap)


def test_select_overflow_and_budget_extremes():
    s = synth.scores(1000, seed=3)
    _select_case(1000, 1, 1000, 1000, s, None)
    _select_case(1000, 1, 1000, 5000, s, None)
    _select_case(1000, 1, 1000, 0, s, synth.pinned_mask(1000, seed=3, frac=0.01))
    _select_case(1000, 1, 1000, 600, s, None, cap=100)


def test_select_segment_device_list():
    keep = torch.full((131072,), -1, dtype=torch.int32, device=DEV)
    nk_dev = torch.zeros(1, dtype=torch.int64, device=DEV)
    n_keep, e = kv.kv_select_segment(131072, 16384, int(0.3 * 131072), 16, keep, nk_dev)
    torch.cuda.synchronize()
    ref = O.select_segment(131072, 16384, int(0.3 * 131072), 16)
    assert e == 39328 and n_keep == len(ref) == int(nk_dev.item())
    assert (keep[:n_keep].cpu().numpy() == ref).all()


# ------------------------------------------------------------------------------ scoring

def _make_score_inputs(w, seed, shuffle, plant=True):
    k, v, bt = synth.kv_cache(w, seed=seed, device="cpu", paged_shuffle=shuffle, extra_pages=2)
    q = synth.window_queries(w, seed=seed)
    if plant:
        synth.plant_heavy_keys(w, k, q, bt, seed=seed)
    return k.to(DEV), v.to(DEV), (bt.to(DEV) if bt is not None else None), q


def _run_score(w, k, v, bt, q, *, policy, item_tokens, state, lse_in=None, **kw):
    n = w.n_tokens
    n_items = -(-n // item_tokens)
    out = dict(mass=torch.zeros(n, device=DEV), lse=torch.zeros((w.n_layers, w.n_q_heads, w.window), device=DEV),
               token_score=torch.zeros(n, device=DEV), item_score=torch.zeros(n_items, device=DEV),
               item_pinned=torch.zeros(n_items, dtype=torch.uint8, device=DEV))
    kv.kv_score(kv.PagedCache(k, v, n, bt), q.to(DEV), policy=policy, window=w.window, item_tokens=item_tokens,
                lse_in=lse_in, **state, **kw, **out)
    torch.cuda.synchronize()
    return {key: t.cpu() for key, t in out.items()}


def _memdecay_state(w, seed):
    ewma, clock = synth.memdecay_state(w, seed)
    b, lam = synth.region_params(seed)
    return dict(region=synth.regions(w, seed), base_prio=b, decay_rate=lam, ewma=ewma, clock=clock)


def _compare_memdecay(w, q, k_logical, st0, dev_state, got, rho, alpha, tau, dt_steps, item_tokens,
                      pinned_regions, n_sink=0, n_recent=0, span_id=None, span_bonus=None):
    ref = O.score_step(np64(q), k_logical, policy="memdecay", region=st0["region"].numpy(),
                       base_prio=np64(st0["base_prio"]), decay_rate=np64(st0["decay_rate"]),
                       rho=f32(rho), alpha=f32(alpha), tau=f32(tau), dt_steps=dt_steps,
                       ewma=np64(st0["ewma"]), clock=st0["clock"].numpy(),
                       span_id=None if span_id is None else span_id.numpy(),
                       span_bonus=None if span_bonus is None else span_bonus.numpy(),
                       pinned_regions=pinned_regions, n_sink=n_sink, n_recent=n_recent,
                       item_tokens=item_tokens)
    assert_rel(np64(got["mass"]), ref["mass"], what="mass")
    assert np.abs(np64(got["lse"]) - ref["lse"]).max() < 1e-5
    boundary = np.abs(ref["abar"] - f32(tau)) <= 1e-5 * f32(tau)
    ok = ~boundary
    assert_rel(np64(dev_state["ewma"])[ok], ref["ewma"][ok], what="ewma")
    assert (dev_state["clock"].numpy()[ok] == ref["clock"][ok]).all()
    assert_rel(np64(got["token_score"])[ok], ref["token_score"][ok], what="token score")
    item_ok = ok if item_tokens == 1 else ~O.page_any(boundary, item_tokens)
    assert_rel(np64(got["item_score"])[item_ok], ref["item_score"][item_ok], what="item score")
    assert (got["item_pinned"].numpy().astype(bool) == ref["item_pinned"]).all()
    return ref, boundary


@pytest.mark.parametrize("name,over,shuffle", [
    ("qwen2.5-1.5b-1layer-n512", {}, False),
    ("qwen2.5-1.5b-1layer-n512", {}, True),
    ("qwen2.5-1.5b-n2048", {}, True),
    ("qwen2.5-1.5b-1layer-n512", dict(n_tokens=1000, window=37, n_q_heads=6, n_kv_heads=2, n_layers=2), True),
    ("qwen2.5-1.5b-1layer-n512", dict(n_tokens=77, window=77, n_q_heads=4, n_kv_heads=4, n_layers=1, system_prefix=5), False),
    ("qwen2.5-1.5b-1layer-n512", dict(n_tokens=5000, window=64, n_q_heads=32, n_kv_heads=8, n_layers=2, system_prefix=64), True),
    ("qwen2.5-1.5b-1layer-n512", dict(n_tokens=9000, window=16, n_q_heads=64, n_kv_heads=2, n_layers=1), False),
])
def test_score_memdecay_parity(name, over, shuffle):
    w = synth.workload(name, **{**over, "n_spans": 24})
    k, v, bt, q = _make_score_inputs(w, seed=11 + w.n_tokens, shuffle=shuffle)
    st0 = _memdecay_state(w, seed=w.n_tokens)
    span_id, span_bonus = synth.spans(w, seed=w.n_tokens, p_needed=0.25)
    dev_state = {key: t.clone() for key, t in st0.items()}
    dev = {key: t.to(DEV) for key, t in dev_state.items()}
    got = _run_score(w, k, v, bt, q, policy="memdecay", item_tokens=w.item_tokens, state=dev,
                     rho=w.rho, alpha=w.alpha, tau=w.tau, dt_steps=3, pinned_regions=1,
                     span_id=span_id.to(DEV), span_bonus=span_bonus.to(DEV))
    dev_state = {key: t.cpu() for key, t in dev.items()}
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    _compare_memdecay(w, q, kl, st0, dev_state, got, w.rho, w.alpha, w.tau, 3, w.item_tokens, 1,
                      span_id=span_id, span_bonus=span_bonus)


def test_score_memdecay_sixteen_steps():
    """State carried across 16 scoring steps with fresh window queries (Qwen2.5-1.5B shape, 512 tokens)."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512")
    k, v, bt, _ = _make_score_inputs(w, seed=5, shuffle=True)
    st = _memdecay_state(w, seed=5)
    dev = {key: t.to(DEV) for key, t in st.items()}
    ref_ewma, ref_clock = np64(st["ewma"]), st["clock"].numpy().astype(np.int64)
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    excluded = np.zeros(w.n_tokens, bool)
    for step in range(16):
        q = synth.window_queries(w, seed=100 + step)
        got = _run_score(w, k, v, bt, q, policy="memdecay", item_tokens=16, state=dev, rho=w.rho,
                         alpha=w.alpha, tau=w.tau, dt_steps=1, pinned_regions=1)
        ref = O.score_step(np64(q), kl, policy="memdecay", region=st["region"].numpy(),
                           base_prio=np64(st["base_prio"]), decay_rate=np64(st["decay_rate"]),
                           rho=f32(w.rho), alpha=f32(w.alpha), tau=f32(w.tau), dt_steps=1,
                           ewma=ref_ewma, clock=ref_clock, pinned_regions=1, item_tokens=16)
        excluded |= np.abs(ref["abar"] - f32(w.tau)) <= 1e-5 * f32(w.tau)
        ok = ~excluded
        assert_rel(np64(dev["ewma"].cpu())[ok], ref["ewma"][ok], what=f"ewma step {step}")
        assert (dev["clock"].cpu().numpy()[ok] == ref["clock"][ok]).all(), step
        assert_rel(np64(got["token_score"])[ok], ref["token_score"][ok], what=f"score step {step}")
        ref_ewma, ref_clock = ref["ewma"], ref["clock"]
    assert excluded.mean() < 0.01


@pytest.mark.parametrize("over,shuffle", [
    (dict(n_tokens=3000, n_layers=2, n_spans=40), True),
    (dict(n_tokens=10_000, n_layers=1, n_spans=200), False),
])
def test_score_h2o_foresight_parity(over, shuffle):
    w = synth.workload("qwen3-8b-n100k", **over)
    k, v, bt, q = _make_score_inputs(w, seed=w.n_tokens, shuffle=shuffle)
    span_id, span_bonus = synth.spans(w, seed=3, p_needed=0.2)
    # tokens outside every span (-1) and ids that name no span of the table get no bonus
    g = torch.Generator().manual_seed(w.n_tokens)
    r = torch.rand(w.n_tokens, generator=g)
    span_id = torch.where(r < 0.05, torch.full_like(span_id, -1), span_id)
    span_id = torch.where((r >= 0.05) & (r < 0.08), span_id + w.n_spans, span_id)
    span_id[:3] = torch.tensor([-2 ** 31, 2 ** 31 - 1, w.n_spans], dtype=torch.int32)
    accum = synth.h2o_state(w, seed=3)
    dev_acc = accum.to(DEV)
    got = _run_score(w, k, v, bt, q, policy="h2o", item_tokens=1, state=dict(accum=dev_acc),
                     span_id=span_id.to(DEV), span_bonus=span_bonus.to(DEV), n_sink=w.n_sink,
                     n_recent=w.n_recent)
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    ref = O.score_step(np64(q), kl, policy="h2o", accum=np64(accum), span_id=span_id.numpy(),
                       span_bonus=span_bonus.numpy(), n_sink=w.n_sink,
                       n_recent=w.n_recent)
    assert_rel(np64(got["mass"]), ref["mass"], what="mass")
    assert_rel(np64(dev_acc.cpu()), ref["accum"], what="accum")
    assert_rel(np64(got["item_score"]), ref["item_score"], what="score")
    assert (got["item_pinned"].numpy().astype(bool) == ref["item_pinned"]).all()
    assert (span_bonus > 0).any() and (span_id < 0).any() and (span_id >= w.n_spans).any()


# 1,000 tokens: the mass pass combines the LSE itself; 40,000: 64 key chunks, so a
# separate combine launch does it (and clears the status word)
@pytest.mark.parametrize("n_tokens", [1000, 40_000])
def test_score_bad_region_labels_are_reported(n_tokens):
    """Labels at or above n_regions name no region (b = lambda = 0, no region pin) and set
    KV_STATUS_BAD_REGION; a clean row leaves the status word at 0."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=n_tokens, n_layers=2, window=32)
    k, v, bt, q = _make_score_inputs(w, seed=44, shuffle=True)
    st0 = _memdecay_state(w, seed=44)
    n_regions = int(st0["base_prio"].numel())
    bad = torch.zeros(w.n_tokens, dtype=torch.bool)
    bad[::37] = True
    region = st0["region"].clone()
    region[bad] = torch.randint(n_regions, 256, (int(bad.sum()),), generator=torch.Generator().manual_seed(1),
                                dtype=torch.int32).to(torch.uint8)
    region[5] = 255
    st_bad = dict(st0, region=region)
    for state, want in ((st0, 0), (st_bad, kv.KV_STATUS_BAD_REGION)):
        dev = {key: t.clone().to(DEV) for key, t in state.items()}
        status = torch.full((1,), 0x55, dtype=torch.int32, device=DEV)
        got = _run_score(w, k, v, bt, q, policy="memdecay", item_tokens=1, state=dev, rho=w.rho,
                         alpha=w.alpha, tau=w.tau, dt_steps=2, pinned_regions=0b11, status=status)
        assert int(status.item()) == want
        dev_state = {key: t.cpu() for key, t in dev.items()}
        kl = _paged_to_logical(k, bt, 16, w.n_tokens)
        _compare_memdecay(w, q, kl, state, dev_state, got, w.rho, w.alpha, w.tau, 2, 1, 0b11)


def test_score_with_supplied_lse():
    """Single-pass mode: LSE given by the attention backend (ActKV Sec. 7.1)."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=3000, n_layers=2, window=48)
    k, v, bt, q = _make_score_inputs(w, seed=9, shuffle=True)
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    mass, lse = O.attention_mass(np64(q), kl)
    acc = torch.zeros(w.n_tokens, device=DEV)
    got = _run_score(w, k, v, bt, q, policy="h2o", item_tokens=1, state=dict(accum=acc),
                     lse_in=torch.from_numpy(lse).float().to(DEV))
    assert_rel(np64(got["mass"]), mass, what="mass with supplied LSE")


@pytest.mark.parametrize("hq,hkv,window,n_tokens,n_layers", [
    (4, 4, 24, 700, 2),      # G = 1: equals the sum
    (4, 2, 40, 1500, 1),     # G = 2
    (6, 2, 33, 2000, 2),     # G = 3, padded to 4
    (32, 8, 64, 5000, 2),    # G = 4: Qwen3-8B / Mistral-7B heads, 256 rows
    (28, 4, 32, 3000, 1),    # G = 7, padded to 8 (Qwen2.5-7B heads)
    (40, 8, 50, 2500, 1),    # G = 5, padded to 8: 400 rows, two row groups
    (32, 2, 20, 1800, 1),    # G = 16: 320 rows
    (32, 1, 16, 1300, 1),    # G = 32: 512 rows
    # grids small enough that the mass pass combines the LSE itself, with two row groups
    (32, 2, 20, 600, 1),     # G = 16: 320 rows, 10 key chunks
    (40, 8, 50, 700, 1),     # G = 5, padded to 8: 400 rows, 11 key chunks
])
def test_score_max_group_parity(hq, hkv, window, n_tokens, n_layers):
    """ActKV's aggregation (Sec. 7.1, Algorithm 3): per KV head the maximum over its
    query heads of exp(s - LSE), against the oracle; MemDecay divides by L*Hkv*W."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=n_tokens, window=window, n_q_heads=hq, n_kv_heads=hkv,
                       n_layers=n_layers)
    k, v, bt, q = _make_score_inputs(w, seed=31 + n_tokens, shuffle=True)
    st0 = _memdecay_state(w, seed=n_tokens)
    dev = {key: t.clone().to(DEV) for key, t in st0.items()}
    got = _run_score(w, k, v, bt, q, policy="memdecay", item_tokens=w.item_tokens, state=dev,
                     rho=w.rho, alpha=w.alpha, tau=w.tau, dt_steps=2, pinned_regions=1,
                     aggregate="max_group")
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    ref = O.score_step(np64(q), kl, policy="memdecay", region=st0["region"].numpy(),
                       base_prio=np64(st0["base_prio"]), decay_rate=np64(st0["decay_rate"]),
                       rho=f32(w.rho), alpha=f32(w.alpha), tau=f32(w.tau), dt_steps=2,
                       ewma=np64(st0["ewma"]), clock=st0["clock"].numpy(), pinned_regions=1,
                       item_tokens=w.item_tokens, aggregate="max_group")
    assert_rel(np64(got["mass"]), ref["mass"], what="group-max score")
    assert np.abs(np64(got["lse"]) - ref["lse"]).max() < 1e-5
    ok = np.abs(ref["abar"] - f32(w.tau)) > 1e-5 * f32(w.tau)
    assert_rel(np64(dev["ewma"].cpu())[ok], ref["ewma"][ok], what="ewma")
    assert (dev["clock"].cpu().numpy()[ok] == ref["clock"][ok]).all()
    assert_rel(np64(got["token_score"])[ok], ref["token_score"][ok], what="token score")
    if hq == hkv:   # one head per group: the same numbers as the sum
        s = _run_score(w, k, v, bt, q, policy="h2o", item_tokens=1,
                       state=dict(accum=torch.zeros(w.n_tokens, device=DEV)))
        assert torch.equal(s["mass"], got["mass"])


# 1,000 tokens (16 key chunks): the mass pass reads the supplied LSE itself; 2,600 and
# 40,000 (21 and 63 chunks): the combine launch converts it first
@pytest.mark.parametrize("aggregate,shift,n_tokens", [("sum", 0.0, 1000), ("max_group", 0.0, 1000),
                                                      ("max_group", 0.3, 1000), ("sum", 0.0, 2600),
                                                      ("max_group", 0.3, 2600), ("sum", 0.0, 40_000),
                                                      ("max_group", 0.3, 40_000)])
def test_score_supplied_lse_both_modes(aggregate, shift, n_tokens):
    """A supplied LSE is used as given (ActKV Sec. 7.1): also when it is not the keys' own."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=n_tokens, n_layers=2, window=40, n_q_heads=12,
                       n_kv_heads=4)
    k, v, bt, q = _make_score_inputs(w, seed=17, shuffle=True)
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    _, lse = O.attention_mass(np64(q), kl)
    lse_in = (lse + shift).astype(np.float32)
    fn = O.attention_mass if aggregate == "sum" else O.attention_score_max_group
    mass, _ = fn(np64(q), kl, lse=lse_in.astype(np.float64))
    got = _run_score(w, k, v, bt, q, policy="h2o", item_tokens=1,
                     state=dict(accum=torch.zeros(w.n_tokens, device=DEV)),
                     lse_in=torch.from_numpy(lse_in).to(DEV), aggregate=aggregate)
    assert_rel(np64(got["mass"]), mass, what=f"{aggregate} with supplied LSE")
    assert np.abs(np64(got["lse"]) - lse_in).max() < 1e-5


@pytest.mark.parametrize("ps", [1, 2, 4, 8, 64, 1024])
def test_score_page_sizes(ps):
    """Every supported page size: the scoring kernels take the per-lane address path
    below 4 tokens per page and wave-uniform pages from 4 on."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=3000, window=40, n_q_heads=8, n_kv_heads=2, n_layers=2, page_size=ps)
    k, v, bt = synth.kv_cache(w, seed=ps, device="cpu", paged_shuffle=True, extra_pages=2)
    q = synth.window_queries(w, seed=ps)
    acc = torch.zeros(w.n_tokens, device=DEV)
    got = _run_score(w, k.to(DEV), v.to(DEV), bt.to(DEV), q, policy="h2o", item_tokens=1,
                     state=dict(accum=acc))
    kl = O.gather_logical(np64(k), bt.numpy(), ps, w.n_tokens)
    mass, lse = O.attention_mass(np64(q), kl)
    assert_rel(np64(got["mass"]), mass, what=f"mass, page {ps}")
    assert np.abs(np64(got["lse"]) - lse).max() < 1e-5


@pytest.mark.parametrize("src_ps,dst_ps", [(1, 1024), (1024, 1), (2, 64), (64, 4)])
def test_compact_page_sizes(src_ps, dst_ps):
    nl, hkv, n, n_keep = 2, 2, 2500, 700
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=nl, n_kv_heads=hkv, n_q_heads=hkv, n_tokens=n, page_size=src_ps)
    k, v, bt = synth.kv_cache(w, seed=src_ps + dst_ps, device=DEV, paged_shuffle=True, extra_pages=2)
    g = torch.Generator().manual_seed(src_ps * 7 + dst_ps)
    keep = torch.sort(torch.randperm(n, generator=g)[:n_keep])[0].to(torch.int32)
    old_pos = torch.arange(n, dtype=torch.int32) + 5000
    n_dst_pages = -(-n_keep // dst_ps)
    dk = torch.zeros((nl, n_dst_pages + 1, dst_ps, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    dbt = torch.randperm(n_dst_pages + 1, generator=g)[:n_dst_pages].to(torch.int32).to(DEV)
    newp = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, n, bt), kv.PagedCache(dk, dv, n_keep, dbt), keep.to(DEV), None,
                         n_keep, old_pos.to(DEV), newp, renumber_base=0, rope_theta=1e6)
    torch.cuda.synchronize()
    kl = O.gather_logical(np64(k), bt.cpu().numpy(), src_ps, n)
    vl = O.gather_logical(np64(v), bt.cpu().numpy(), src_ps, n)
    rk, rv, rpos = O.compact_rerope(kl, vl, keep.numpy(), old_pos.numpy(), 0, 1e6)
    gk = unpage(np64(dk), dbt.cpu().numpy(), dst_ps, n_keep)
    gv = unpage(np64(dv), dbt.cpu().numpy(), dst_ps, n_keep)
    assert (newp.cpu().numpy() == rpos).all()
    assert (gv == rv).all()
    assert_bf16_within_1ulp(gk, rk, f"K, pages {src_ps}->{dst_ps}")


def test_pipeline_end_to_end_config2():
    """score -> select -> compact on the GPU against the oracle pipeline (Qwen2.5-1.5B, 28 layers, 2,048 tokens)."""
    w = synth.workload("qwen2.5-1.5b-n2048")
    k, v, bt, q = _make_score_inputs(w, seed=21, shuffle=True)
    st0 = _memdecay_state(w, seed=21)
    dev = {key: t.to(DEV) for key, t in st0.items()}
    got = _run_score(w, k, v, bt, q, policy="memdecay", item_tokens=16, state=dev, rho=w.rho,
                     alpha=w.alpha, tau=w.tau, dt_steps=1, pinned_regions=1)
    keep = torch.zeros(w.budget_tokens + 64, dtype=torch.int32, device=DEV)
    n_keep = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_select(got["item_score"].to(DEV), got["item_pinned"].to(DEV), 16, w.n_tokens, w.budget_items,
                 keep, n_keep)
    kl = _paged_to_logical(k, bt, 16, w.n_tokens)
    ref = O.score_step(np64(q), kl, policy="memdecay", region=st0["region"].numpy(),
                       base_prio=np64(st0["base_prio"]), decay_rate=np64(st0["decay_rate"]),
                       rho=f32(w.rho), alpha=f32(w.alpha), tau=f32(w.tau), dt_steps=1,
                       ewma=np64(st0["ewma"]), clock=st0["clock"].numpy(), pinned_regions=1, item_tokens=16)
    items, _ = O.select_items(ref["item_score"], ref["item_pinned"], w.budget_items)
    torch.cuda.synchronize()
    nk = int(n_keep.item())
    got_items = np.unique(keep[:nk].cpu().numpy() // 16)
    diff = set(items.tolist()) ^ set(got_items.tolist())
    if diff:
        unp = ~ref["item_pinned"]
        thr = np.sort(ref["item_score"][unp])[::-1][w.budget_items - ref["item_pinned"].sum() - 1]
        for d in diff:
            assert abs(ref["item_score"][d] - thr) <= 1e-5 * abs(thr), d
    # compaction of the GPU keep list, renumbered to 0..n-1
    dk = torch.zeros((w.n_layers, w.budget_tokens // 16 + 4, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    pos = torch.arange(w.n_tokens, dtype=torch.int32, device=DEV)
    newp = torch.zeros(w.budget_tokens + 64, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, w.n_tokens, bt), kv.PagedCache(dk, dv, w.budget_tokens + 64),
                         keep, n_keep, w.budget_tokens + 64, pos, newp, renumber_base=0,
                         rope_theta=w.rope_theta, limit=8192)
    torch.cuda.synchronize()
    keep_np = keep[:nk].cpu().numpy()
    rk, rv, _ = O.compact_rerope(kl, _paged_to_logical(v, bt, 16, w.n_tokens), keep_np, np.arange(w.n_tokens),
                                 0, w.rope_theta)
    gk = np64(dk).reshape(w.n_layers, -1, 2, 128)[:, :nk]
    gv = np64(dv).reshape(w.n_layers, -1, 2, 128)[:, :nk]
    assert (gv == rv).all()
    assert_bf16_within_1ulp(gk, rk, "pipeline K")


# ------------------------------------------------------------------------------ full sizes

@pytest.fixture(scope="module")
def qwen3_100k():
    w = synth.workload("qwen3-8b-n100k")
    k, v, _ = synth.kv_cache(w, seed=0, device=DEV)
    q = synth.window_queries(w, seed=0, device=DEV)
    yield w, k, v, q
    del k, v
    torch.cuda.empty_cache()


def test_full_size_qwen3_100k_score_properties(qwen3_100k):
    """Launch configuration of the benchmark: 36 layers, 32/8 heads, N = 100,000."""
    w, k, v, q = qwen3_100k
    span_id, span_bonus = synth.spans(w, seed=0)
    acc = torch.zeros(w.n_tokens, device=DEV)
    got = _run_score(w, k, v, None, q, policy="h2o", item_tokens=1, state=dict(accum=acc),
                     span_id=span_id.to(DEV), span_bonus=span_bonus.to(DEV), n_sink=4, n_recent=128)
    mass = np64(got["mass"])
    total = w.n_layers * w.n_q_heads * w.window
    assert abs(mass.sum() / total - 1) < 1e-5          # each query's softmax row sums to 1
    assert (mass > 0).all()
    # sampled LSE rows against the oracle's definition over all 100K keys
    g = torch.Generator().manual_seed(0)
    for _ in range(6):
        layer = int(torch.randint(0, w.n_layers, (1,), generator=g))
        h = int(torch.randint(0, w.n_q_heads, (1,), generator=g))
        wi = int(torch.randint(0, w.window, (1,), generator=g))
        kk = np64(k[layer, :, :, h // 4, :].reshape(-1, 128)[: w.n_tokens])
        qq = np64(q[layer, wi, h])
        qpos = w.n_tokens - w.window + wi
        s = (kk[: qpos + 1] @ qq) / math.sqrt(128)
        m = s.max()
        ref = m + math.log(np.exp(s - m).sum())
        assert abs(float(got["lse"][layer, h, wi]) - ref) < 1e-5


def test_full_size_qwen3_100k_two_layer_mass(qwen3_100k):
    """Full N with a 2-layer slice of the cache: every token's mass against the oracle."""
    w, k, v, q = qwen3_100k
    w2 = synth.workload("qwen3-8b-n100k", n_layers=2)
    k2, v2, q2 = k[:2].contiguous(), v[:2].contiguous(), q[:2].contiguous()
    acc = torch.zeros(w.n_tokens, device=DEV)
    got = _run_score(w2, k2, v2, None, q2, policy="h2o", item_tokens=1, state=dict(accum=acc))
    kl = np64(k2).reshape(2, -1, 8, 128)[:, : w.n_tokens]
    mass, lse = O.attention_mass(np64(q2), kl)
    assert_rel(np64(got["mass"]), mass, what="mass at N=100K")
    assert np.abs(np64(got["lse"]) - lse).max() < 1e-5


@pytest.mark.parametrize("aggregate", ["sum", "max_group"])
def test_full_size_qwen3_100k_mass_is_additive_over_layers(qwen3_100k, aggregate):
    """Every token's mass at the benchmark's launch configuration (36 layers: a few large key
    chunks per (layer, KV head)) equals the sum of 18 two-layer runs (many small chunks, the
    configuration the oracle checks token by token above and, for the group maximum, at
    smaller sizes).  Either aggregate is a sum over layers, so this holds exactly in real
    arithmetic; each side is within RTOL of it, hence 2*RTOL.  Every row's LSE must agree
    the same way."""
    w, k, v, q = qwen3_100k
    acc = torch.zeros(w.n_tokens, device=DEV)
    full = _run_score(w, k, v, None, q, policy="h2o", item_tokens=1, state=dict(accum=acc),
                      aggregate=aggregate)
    w2 = synth.workload("qwen3-8b-n100k", n_layers=2)
    total = np.zeros(w.n_tokens)
    for l0 in range(0, w.n_layers, 2):
        acc.zero_()
        part = _run_score(w2, k[l0:l0 + 2].contiguous(), v[l0:l0 + 2].contiguous(), None,
                          q[l0:l0 + 2].contiguous(), policy="h2o", item_tokens=1, state=dict(accum=acc),
                          aggregate=aggregate)
        total += np64(part["mass"])
        # two device runs, each within 1e-5 of the exact LSE
        assert np.abs(np64(full["lse"][l0:l0 + 2]) - np64(part["lse"])).max() < 2e-5, l0
    assert_rel(np64(full["mass"]), total, rtol=2 * RTOL, what=f"36-layer {aggregate} mass vs 2-layer runs")


def _rerope_chunks(k_rows, v_rows, old_kept, theta, step=512):
    """The oracle's compaction of already gathered rows (rank r holds source keep[r] with
    old position old_kept[r]), renumbered to 0..n-1, in rank chunks to bound memory."""
    n = k_rows.shape[1]
    ks, vs, ps = [], [], []
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        rk, rv, rp = O.compact_rerope(k_rows[:, r0:r1], v_rows[:, r0:r1], np.arange(r1 - r0),
                                      old_kept[r0:r1], r0, theta)      # ranks r0.. renumber to r0..
        ks.append(rk)
        vs.append(rv)
        ps.append(rp)
    return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1), np.concatenate(ps)


def test_full_size_qwen3_100k_bench_step(qwen3_100k):
    """The benchmark's own step at full size (Qwen3-8B shape, 36 layers, N = 100,000):
    H2O + foresight scoring, selection of 2,048 tokens with 4 sinks and 128 recent pinned,
    compaction with renumbering under L = 8,192 and the metadata it carries.  Checked:
    every token's score is its mass plus the oracle's bonus, the pins follow the rules, the
    keep list equals the oracle's selection on the device's own scores bit for bit, and all
    2,048 compacted ranks (V, unrotated and rotated K, positions, metadata) match the
    oracle's compaction of the kept rows."""
    w, k, v, q = qwen3_100k
    N, B = w.n_tokens, w.budget_tokens
    span_id, span_bonus = synth.spans(w, seed=0)
    accum = torch.zeros(N, device=DEV)
    mass = torch.zeros(N, device=DEV)
    tok = torch.zeros(N, device=DEV)
    item_score = torch.zeros(N, device=DEV)
    item_pinned = torch.zeros(N, dtype=torch.uint8, device=DEV)
    src = kv.PagedCache(k, v, N)
    kv.kv_score(src, q, policy="h2o", window=w.window, item_tokens=1, accum=accum, span_id=span_id.to(DEV),
                span_bonus=span_bonus.to(DEV), n_sink=w.n_sink, n_recent=w.n_recent,
                mass=mass, token_score=tok, item_score=item_score, item_pinned=item_pinned)
    keep = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    n_keep = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.full((1,), 9, dtype=torch.int32, device=DEV)
    kv.kv_select(item_score, item_pinned, 1, N, B, keep, n_keep, status)
    dk = torch.zeros((w.n_layers, B // 16, 16, 8, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    old_pos = torch.arange(N, dtype=torch.int32, device=DEV)
    new_pos = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    dst_accum = torch.zeros(B, device=DEV)
    dst_span = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(src, kv.PagedCache(dk, dv, B), keep, n_keep, B, old_pos, new_pos, renumber_base=0,
                         rope_theta=w.rope_theta, limit=w.limit,
                         meta=[(accum, dst_accum), (span_id.to(DEV), dst_span)])
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(n_keep.item()) == B
    # scores: H2O from a zero accumulator is the mass, plus the span bonus
    bonus = O.token_bonus(span_id.numpy(), span_bonus.numpy())
    assert_rel(np64(tok), np64(mass) + bonus, what="score = mass + bonus")
    assert torch.equal(tok, item_score) and torch.equal(accum, mass)
    pin = O.pinned_tokens(N, n_sink=w.n_sink, n_recent=w.n_recent)
    assert (item_pinned.cpu().numpy().astype(bool) == pin).all()
    want, st = O.select_items(np64(item_score), pin, B)
    kept = keep.cpu().numpy().astype(np.int64)
    assert st == 0 and (kept == want).all(), "keep list differs from the oracle's selection"
    # every compacted rank against the oracle
    kl = k.reshape(w.n_layers, -1, 8, 128)[:, keep.long()]
    vl = v.reshape(w.n_layers, -1, 8, 128)[:, keep.long()]
    rk, rv, rpos = _rerope_chunks(np64(kl), np64(vl), kept, w.rope_theta)
    gk = np64(dk).reshape(w.n_layers, B, 8, 128)
    gv = np64(dv).reshape(w.n_layers, B, 8, 128)
    assert (new_pos.cpu().numpy() == rpos).all() and (rpos == np.arange(B)).all()
    assert (gv == rv).all(), "V must be bit-exact"
    still = kept == np.arange(B)
    assert (gk[:, still] == rk[:, still]).all()
    assert_bf16_within_1ulp(gk, rk, "K, all 2,048 ranks")
    assert (dst_accum.cpu() == accum.cpu()[kept]).all() and (dst_span.cpu() == span_id[kept]).all()


def test_long_single_head_row_many_chunks():
    """One layer, one KV head (two query heads, W = 4) over 2^21 + 37 tokens behind a shuffled
    block table: every scoring pass splits the row into hundreds of key chunks of the one
    (layer, KV head), so the LSE combine takes that many partials per row and the selection
    runs on two million items over its largest block count.  LSE, every token's mass and
    score against the oracle; the keep list bit-exact against the oracle's selection on the
    device's own scores; all kept ranks' K within 1 ulp and V, positions exact."""
    N = (1 << 21) + 37
    w = synth.workload("qwen3-8b-n100k", n_layers=1, n_q_heads=2, n_kv_heads=1, window=4, n_tokens=N)
    k, v, bt = synth.kv_cache(w, seed=5, device=DEV, paged_shuffle=True, extra_pages=3)
    q = synth.window_queries(w, seed=5, device=DEV)
    acc0 = torch.rand(N, generator=torch.Generator().manual_seed(5)) * 1e-5   # comparable with the mass
    acc = acc0.to(DEV)
    got = _run_score(w, k, v, bt, q, policy="h2o", item_tokens=1, state=dict(accum=acc), n_sink=4, n_recent=128)
    kl = _paged_to_logical(k, bt, 16, N)
    ref = O.score_step(np64(q), kl, policy="h2o", accum=np64(acc0), n_sink=4, n_recent=128, item_tokens=1)
    assert np.abs(np64(got["lse"]) - ref["lse"]).max() < 1e-5
    assert_rel(np64(got["mass"]), ref["mass"], what="mass")
    assert_rel(np64(acc), ref["accum"], what="accum")
    assert_rel(np64(got["item_score"]), ref["item_score"], what="item score")
    assert (got["item_pinned"].numpy().astype(bool) == ref["item_pinned"]).all()
    # selection on the device's own scores, bit-exact
    B = 2048
    keep = torch.zeros(B, dtype=torch.int32, device=DEV)
    n_keep = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_select(got["item_score"].to(DEV), got["item_pinned"].to(DEV), 1, N, B, keep, n_keep)
    items, _ = O.select_items(np64(got["item_score"]), got["item_pinned"].numpy(), B)
    torch.cuda.synchronize()
    nk = int(n_keep.item())
    keep_np = keep[:nk].cpu().numpy()
    assert nk == B and (keep_np == items).all()
    # compaction of every kept rank, renumbered from 0
    dk = torch.zeros((1, B // 16, 16, 1, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    newp = torch.zeros(B, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, N, bt), kv.PagedCache(dk, dv, B), keep, n_keep, B, pos, newp,
                         renumber_base=0, rope_theta=w.rope_theta, limit=0)
    torch.cuda.synchronize()
    rk, rv, rpos = O.compact_rerope(kl, _paged_to_logical(v, bt, 16, N), keep_np, np.arange(N), 0, w.rope_theta)
    assert (newp.cpu().numpy() == rpos).all()
    assert (np64(dv).reshape(1, B, 1, 128) == rv).all()
    assert_bf16_within_1ulp(np64(dk).reshape(1, B, 1, 128), rk, "long row K")


def test_full_size_mistral_131k_segment():
    """Mistral-7B shape at full size (32 layers, 131,072 tokens, 16,384-token prefix, 30%
    evicted): in-place segment eviction + re-rotation as bench.py --extras runs it.  Every
    one of the 91,744 ranks of the first and the last layer against the oracle's
    compaction of the original rows, and sampled ranks of every layer."""
    w = synth.workload("mistral-7b-n131072-segment")
    N, NL = w.n_tokens, w.n_layers
    k, v, _ = synth.kv_cache(w, seed=0, device=DEV)
    n_keep, e = kv.kv_select_segment(N, w.segment_prefix, int(w.segment_frac * N), 16)
    assert (n_keep, e) == (N - 39_328, 39_328)
    keep = O.select_segment(N, w.segment_prefix, int(w.segment_frac * N), 16)
    assert len(keep) == n_keep
    kf, vf = k.reshape(NL, -1, 8, 128), v.reshape(NL, -1, 8, 128)
    layers = [0, NL - 1]
    k_edge = kf[layers][:, :N].cpu()
    v_edge = vf[layers][:, :N].cpu()
    g = torch.Generator().manual_seed(3)
    ranks = sorted(set([0, w.segment_prefix - 1, w.segment_prefix, w.segment_prefix + e - 1, n_keep - 1]
                       + torch.randint(0, n_keep, (40,), generator=g).tolist()))
    srcs = keep[ranks]
    srcs_d = torch.from_numpy(srcs).to(DEV)
    ks_all, vs_all = np64(kf[:, srcs_d]), np64(vf[:, srcs_d])
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    kv.kv_compact_segment_inplace(kv.PagedCache(k, v, N), w.segment_prefix, e, pos, renumber_base=0,
                                  rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    assert (pos[:n_keep].cpu().numpy() == np.arange(n_keep)).all()
    # first and last layer, every rank
    gk = kf[layers][:, :n_keep].cpu()
    gv = vf[layers][:, :n_keep].cpu()
    step = 8192
    for r0 in range(0, n_keep, step):
        r1 = min(n_keep, r0 + step)
        idx = torch.from_numpy(keep[r0:r1])
        rk, rv, rp = O.compact_rerope(np64(k_edge[:, idx]), np64(v_edge[:, idx]), np.arange(r1 - r0),
                                      keep[r0:r1], r0, w.rope_theta)
        assert (rp == np.arange(r0, r1)).all()
        assert (np64(gv[:, r0:r1]) == rv).all(), r0
        got = np64(gk[:, r0:r1])
        moved = keep[r0:r1] != np.arange(r0, r1)
        assert (got[:, ~moved] == rk[:, ~moved]).all(), r0
        assert_bf16_within_1ulp(got, rk, f"K ranks {r0}..{r1}")
    # sampled ranks of every layer
    delta = np.array(ranks) - srcs
    rk = O.bf16_round(O.rope_rotate(ks_all, delta[None, :, None], w.rope_theta))
    rk[:, delta == 0] = ks_all[:, delta == 0]
    assert (np64(vf[:, ranks]) == vs_all).all()
    assert_bf16_within_1ulp(np64(kf[:, ranks]), rk, "K at N=131K, all layers")
    del k, v
    torch.cuda.empty_cache()


def test_full_size_qwen3_1m_step_properties():
    """Qwen3-8B shape at 1,000,000 tokens (147 GB), the step bench.py --extras times:
    MemDecay page scoring, page selection, compaction.  The oracle cannot score 1M keys
    for every row, so: softmax rows sum to one, sampled LSE rows over all keys, the
    selection against the oracle on the same page scores, sampled compacted keys, and
    every token's mass against the sum of two-layer runs."""
    w = synth.workload("qwen3-8b-n1m")
    N = w.n_tokens
    k, v, _ = synth.kv_cache(w, seed=0, device=DEV)
    q = synth.window_queries(w, seed=0, device=DEV)
    ewma, clock = synth.memdecay_state(w, seed=0)
    b_r, lam = synth.region_params(0)
    sid, sbonus = synth.spans(w, seed=0)
    n_items = -(-N // 16)
    item_score = torch.zeros(n_items, device=DEV)
    item_pinned = torch.zeros(n_items, dtype=torch.uint8, device=DEV)
    mass = torch.zeros(N, device=DEV)
    lse = torch.zeros((w.n_layers, w.n_q_heads, w.window), device=DEV)
    src = kv.PagedCache(k, v, N)
    kv.kv_score(src, q, policy="memdecay", window=w.window, item_tokens=16, rho=w.rho, alpha=w.alpha,
                tau=w.tau, dt_steps=1, region=synth.regions(w, seed=0).to(DEV), base_prio=b_r.to(DEV),
                decay_rate=lam.to(DEV), ewma=ewma.to(DEV), clock=clock.to(DEV), span_id=sid.to(DEV),
                span_bonus=sbonus.to(DEV), n_sink=w.n_sink, n_recent=w.n_recent,
                pinned_regions=1, mass=mass, lse=lse, item_score=item_score, item_pinned=item_pinned)
    B = w.budget_tokens
    keep = torch.zeros(B, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kv_select(item_score, item_pinned, 16, N, B // 16, keep, nk, status)
    dk = torch.zeros((w.n_layers, B // 16, 16, 8, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    newp = torch.zeros(B, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(src, kv.PagedCache(dk, dv, B), keep, nk, B, pos, newp, renumber_base=0,
                         rope_theta=w.rope_theta, limit=w.limit)
    torch.cuda.synchronize()
    m = np64(mass)
    assert abs(m.sum() / (w.n_layers * w.n_q_heads * w.window) - 1) < 1e-5 and (m > 0).all()
    g = torch.Generator().manual_seed(5)
    for _ in range(3):
        layer = int(torch.randint(0, w.n_layers, (1,), generator=g))
        h = int(torch.randint(0, w.n_q_heads, (1,), generator=g))
        wi = int(torch.randint(0, w.window, (1,), generator=g))
        qpos = N - w.window + wi
        kk = np64(k[layer, :, :, h // 4, :].reshape(-1, 128)[: qpos + 1])
        s = (kk @ np64(q[layer, wi, h])) / math.sqrt(128)
        mx = s.max()
        assert abs(float(lse[layer, h, wi]) - (mx + math.log(np.exp(s - mx).sum()))) < 1e-5
    assert int(status.item()) == 0 and int(nk.item()) == B
    # pinned pages from the inputs (oracle definition), then the keep list against the
    # oracle's selection on the device's own 62,500 page scores, bit for bit
    tok_pin = O.pinned_tokens(N, region=synth.regions(w, seed=0).numpy(), pinned_regions=1,
                              n_sink=w.n_sink, n_recent=w.n_recent)
    pin = O.page_any(tok_pin, 16)
    assert (item_pinned.cpu().numpy().astype(bool) == pin).all()
    want_pages, st = O.select_items(np64(item_score), pin, B // 16)
    assert st == 0
    assert (keep.cpu().numpy() == O.expand_items(want_pages, 16, N)).all(), "1M-token keep list"
    ranks = sorted(set([0, B - 1] + torch.randint(0, B, (24,), generator=g).tolist()))
    srcs = keep.cpu().long()[ranks]
    kf = k.reshape(w.n_layers, -1, 8, 128)
    ks = np64(kf[:, srcs.to(DEV)])
    rk = O.bf16_round(O.rope_rotate(ks, (np.array(ranks) - srcs.numpy())[None, :, None], w.rope_theta))
    gk = np64(dk.reshape(w.n_layers, -1, 8, 128)[:, ranks])
    moved = np.array(ranks) != srcs.numpy()
    assert (gk[:, ~moved] == ks[:, ~moved]).all()
    assert_bf16_within_1ulp(gk[:, moved], rk[:, moved], "K at N=1M")
    del dk, dv
    # every token's mass (and every row's LSE) at this launch configuration equals the sum
    # over 18 two-layer runs, which split the keys into other chunks: mass is additive over
    # layers, each side is within RTOL of the exact value, hence 2*RTOL
    w2 = synth.workload("qwen3-8b-n1m", n_layers=2)
    acc = torch.zeros(N, device=DEV)
    total = np.zeros(N)
    for l0 in range(0, w.n_layers, 2):
        acc.zero_()
        part = _run_score(w2, k[l0:l0 + 2].contiguous(), v[l0:l0 + 2].contiguous(), None,
                          q[l0:l0 + 2].contiguous(), policy="h2o", item_tokens=1, state=dict(accum=acc))
        total += np64(part["mass"])
        # two device runs, each within 1e-5 of the exact LSE
        assert np.abs(np64(lse[l0:l0 + 2]) - np64(part["lse"])).max() < 2e-5, l0
    assert_rel(m, total, rtol=2 * RTOL, what="1M-token mass vs sum of 2-layer runs")
    del k, v
    torch.cuda.empty_cache()


def test_degenerate_sizes():
    """One token, one query, one head: LSE is the single logit and the mass is one per
    (layer, head, query); a single item is selected; an empty keep count moves nothing."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=1, window=1, n_q_heads=1, n_kv_heads=1, n_layers=2)
    k, v, _ = synth.kv_cache(w, seed=1, device="cpu")
    q = synth.window_queries(w, seed=1)
    acc = torch.zeros(1, device=DEV)
    got = _run_score(w, k.to(DEV), v.to(DEV), None, q, policy="h2o", item_tokens=1, state=dict(accum=acc))
    s = np.einsum("ld,ld->l", np64(q)[:, 0, 0], np64(k)[:, 0, 0, 0]) / math.sqrt(128)
    assert np.abs(np64(got["lse"]).reshape(-1) - s).max() < 1e-5
    assert abs(float(got["mass"][0]) - 2.0) <= RTOL * 2.0
    keep = torch.full((4,), -1, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_select(got["item_score"].to(DEV), None, 1, 1, 1, keep, nk)
    torch.cuda.synchronize()
    assert int(nk) == 1 and int(keep[0]) == 0
    # a device count of zero moves nothing
    dk = torch.zeros((2, 1, 16, 1, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    newp = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    zero = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k.to(DEV), v.to(DEV), 1), kv.PagedCache(dk, dv, 1), keep[:1], zero, 1,
                         torch.zeros(1, dtype=torch.int32, device=DEV), newp, renumber_base=3)
    torch.cuda.synchronize()
    assert (dk == 0).all() and int(newp[0]) == -5


def test_score_bit_reproducible():
    """Every reduction has a fixed order: two runs give identical bits."""
    w = synth.workload("qwen2.5-1.5b-1layer-n512", n_tokens=6000, window=64, n_q_heads=32, n_kv_heads=8, n_layers=2)
    k, v, bt, q = _make_score_inputs(w, seed=77, shuffle=True)
    outs = []
    for _ in range(2):
        acc = torch.zeros(w.n_tokens, device=DEV)
        outs.append(_run_score(w, k, v, bt, q, policy="h2o", item_tokens=1, state=dict(accum=acc)))
    for key in ("mass", "lse", "item_score"):
        assert torch.equal(outs[0][key], outs[1][key]), key


def test_compact_skips_out_of_range_keep_entries():
    """Keep entries outside the source row are skipped by the kernels' own bounds checks:
    their ranks are left untouched and every other rank is compacted normally."""
    w = synth.workload("qwen2.5-1.5b-n2048", n_layers=2, n_kv_heads=2, n_q_heads=2, n_tokens=300)
    k, v, _ = synth.kv_cache(w, seed=9, device=DEV)
    keep = torch.arange(0, 300, 10, dtype=torch.int32)          # 30 ranks
    keep[[3, 17]] = torch.tensor([1 << 30, -5], dtype=torch.int32)
    dk = torch.zeros((2, 2, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    newp = torch.full((30,), -9, dtype=torch.int32, device=DEV)
    reg = torch.arange(300, dtype=torch.int32, device=DEV)
    reg_out = torch.full((30,), -1, dtype=torch.int32, device=DEV)
    pos = torch.arange(300, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(k, v, 300), kv.PagedCache(dk, dv, 30), keep.to(DEV), None, 30, pos, newp,
                         renumber_base=-1, rope_theta=1e6, meta=[(reg, reg_out)])
    torch.cuda.synchronize()
    got_v = unpage(np64(dv), None, 16, 30)
    src_v = unpage(np64(v), None, 16, 300)
    ok = [r for r in range(30) if r not in (3, 17)]
    assert (got_v[:, ok] == src_v[:, keep.numpy()[ok]]).all()
    assert (got_v[:, [3, 17]] == 0).all()
    assert (newp.cpu().numpy()[[3, 17]] == -9).all() and (reg_out.cpu().numpy()[[3, 17]] == -1).all()
    assert (newp.cpu().numpy()[ok] == keep.numpy()[ok]).all()
