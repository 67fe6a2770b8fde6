"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test ties one oracle function to something other than itself: a value printed on
a page (fixtures under tests/golden/), a closed form, an invariant, an independent
library routine (torch's bf16 conversion, torch's scaled-dot-product attention, a
Hugging-Face-style rotate-half RoPE, complex multiplication), or brute force.
"""
import itertools
import math
from fractions import Fraction

import hypothesis as hyp
import hypothesis.strategies as st
import numpy as np
import pytest
import torch

import oracle as O
import synth
from conftest import read_golden


# ---------------------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------------------

def test_bf16_round_matches_torch_rne():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(200_000, generator=g) * torch.exp(torch.randn(200_000, generator=g) * 20)
    # include subnormal-range and huge values, exact ties and their neighbours
    ties = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130 * 1.5,
                         2 ** -133 * 0.5, 2 ** -133 * 1.5, 3.3895e38, -0.0, 0.0, 1e-45],
                        dtype=torch.float32)
    x = torch.cat([x.float(), ties])
    ref = x.to(torch.bfloat16).float().double().numpy()
    got = O.bf16_round(x.double().numpy())
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), (x.numpy()[~same][:5], got[~same][:5], ref[~same][:5])
    # signed zero preserved
    assert np.signbit(O.bf16_round(np.array([-0.0])))[0]


def test_bf16_round_ties_to_even_by_hand():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert O.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert O.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    # just above the tie rounds up
    assert O.bf16_round(np.array([1.0 + 2 ** -8 + 2 ** -30]))[0] == 1.0 + 2 ** -7
    # bit pattern round trip
    v = O.bf16_round(np.array([1.5, -2.25, 3.0e-3]))
    assert (O.bf16_from_bits(O.bf16_bits(v)) == v).all()


# ---------------------------------------------------------------------------------------
# Paged layout (ActKV Sec. 2.5)
# ---------------------------------------------------------------------------------------

def test_slot_map_actkv_example():
    gd = read_golden("actkv_slot_map.txt")
    slots = O.slot_map(list(gd["block_table"]), gd["page_size"], gd["n_tokens"])
    assert tuple(slots) == gd["slots"]


def test_gather_logical_follows_block_table():
    rng = np.random.default_rng(3)
    nl, pg, hk, d, n = 2, 4, 2, 3, 13
    n_pages = -(-n // pg)
    bt = rng.permutation(n_pages + 3)[:n_pages]
    paged = rng.standard_normal((nl, n_pages + 3, pg, hk, d))
    logical = O.gather_logical(paged, bt, pg, n)
    for layer in range(nl):
        for j in range(n):
            assert (logical[layer, j] == paged[layer, bt[j // pg], j % pg]).all()
    ident = O.gather_logical(paged, None, pg, n)
    assert (ident[:, 5] == paged[:, 1, 1]).all()


# ---------------------------------------------------------------------------------------
# O1 attention mass
# ---------------------------------------------------------------------------------------

def _rand_qk(rng, nl, w, hq, hkv, d, n):
    q = O.bf16_round(rng.standard_normal((nl, w, hq, d)))
    k = O.bf16_round(rng.standard_normal((nl, n, hkv, d)))
    return q, k


@pytest.mark.parametrize("nl,w,hq,hkv,d,n", [(1, 4, 4, 2, 8, 37), (2, 3, 6, 2, 16, 20),
                                              (1, 1, 2, 1, 4, 5), (2, 5, 8, 8, 8, 5)])
def test_attention_mass_matches_torch_sdpa(nl, w, hq, hkv, d, n):
    """Attention weights recovered from torch's SDPA with identity values (V = I gives
    o = A), GQA via enable_gqa (query head h reads KV head h // G), causal window."""
    rng = np.random.default_rng(nl * 100 + n)
    q, k = _rand_qk(rng, nl, w, hq, hkv, d, n)
    mass, lse = O.attention_mass(q, k)
    qpos = n - w + np.arange(w)
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos[:, None])
    ref = np.zeros(n)
    for layer in range(nl):
        qt = torch.from_numpy(q[layer]).permute(1, 0, 2)[None]          # [1,Hq,W,D]
        kt = torch.from_numpy(k[layer]).permute(1, 0, 2)[None]          # [1,Hkv,N,D]
        vt = torch.eye(n, dtype=torch.float64)[None, None].expand(1, hkv, n, n).contiguous()
        a = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, enable_gqa=True)                 # [1,Hq,W,N]
        ref += a.sum(dim=(0, 1, 2)).numpy()
    np.testing.assert_allclose(mass, ref, rtol=1e-12, atol=1e-14)


def test_attention_mass_sums_to_row_count():
    rng = np.random.default_rng(5)
    q, k = _rand_qk(rng, 3, 7, 6, 3, 16, 50)
    mass, _ = O.attention_mass(q, k)
    assert abs(mass.sum() - 3 * 6 * 7) < 1e-11


def test_attention_mass_equal_keys_closed_form():
    """All keys equal: each query spreads 1/(visible count) over its visible keys."""
    rng = np.random.default_rng(6)
    nl, w, hq, hkv, d, n = 2, 4, 4, 2, 8, 11
    q = rng.standard_normal((nl, w, hq, d))
    k = np.broadcast_to(rng.standard_normal((1, 1, hkv, d)), (nl, n, hkv, d)).copy()
    mass, _ = O.attention_mass(q, k)
    expect = np.zeros(n)
    for wi in range(w):
        qi = n - w + wi
        expect[: qi + 1] += nl * hq / (qi + 1)
    np.testing.assert_allclose(mass, expect, rtol=1e-13)


def test_attention_mass_planted_key_dominates():
    rng = np.random.default_rng(7)
    nl, w, hq, hkv, d, n = 1, 4, 4, 2, 16, 40
    q, k = _rand_qk(rng, nl, w, hq, hkv, d, n)
    for g in range(hkv):
        k[0, 9, g] = 40.0 * q[0, :, 2 * g:2 * g + 2].sum(axis=(0, 1))
    mass, _ = O.attention_mass(q, k)
    assert mass.argmax() == 9 and mass[9] > 0.5 * nl * hq * w


def test_attention_mass_kv_head_permutation_invariant():
    rng = np.random.default_rng(8)
    nl, w, hq, hkv, d, n = 2, 3, 6, 3, 8, 17
    q, k = _rand_qk(rng, nl, w, hq, hkv, d, n)
    perm = np.array([2, 0, 1])
    g = hq // hkv
    qperm = np.concatenate([q[:, :, p * g:(p + 1) * g] for p in perm], axis=2)
    m1, _ = O.attention_mass(q, k)
    m2, _ = O.attention_mass(qperm, k[:, :, perm])
    np.testing.assert_allclose(m1, m2, rtol=1e-13)


def test_lse_matches_logsumexp_scipy():
    from scipy.special import logsumexp
    rng = np.random.default_rng(9)
    q, k = _rand_qk(rng, 1, 3, 2, 1, 8, 12)
    _, lse = O.attention_mass(q, k)
    for wi in range(3):
        qi = 12 - 3 + wi
        s = (q[0, wi, 1] @ k[0, : qi + 1, 0].T) / math.sqrt(8)
        assert abs(lse[0, 1, wi] - logsumexp(s)) < 1e-12


# ---------------------------------------------------------------------------------------
# O1b ActKV aggregation: maximum over each GQA group (Sec. 7.1, Algorithm 3)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("nl,w,hq,hkv,d,n", [(1, 4, 8, 2, 8, 30), (2, 3, 4, 1, 16, 21),
                                              (1, 2, 8, 1, 8, 9)])
def test_max_group_matches_torch_sdpa(nl, w, hq, hkv, d, n):
    """Per (layer, KV head, window query): the maximum over the group's query heads of
    torch's SDPA attention weights (identity values give o = A), summed."""
    rng = np.random.default_rng(nl * 1000 + n)
    q, k = _rand_qk(rng, nl, w, hq, hkv, d, n)
    score, _ = O.attention_score_max_group(q, k)
    qpos = n - w + np.arange(w)
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos[:, None])
    g = hq // hkv
    ref = np.zeros(n)
    for layer in range(nl):
        qt = torch.from_numpy(q[layer]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[layer]).permute(1, 0, 2)[None]
        vt = torch.eye(n, dtype=torch.float64)[None, None].expand(1, hkv, n, n).contiguous()
        a = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, enable_gqa=True)[0]               # [Hq,W,N]
        ref += a.reshape(hkv, g, w, n).max(dim=1).values.sum(dim=(0, 1)).numpy()
    np.testing.assert_allclose(score, ref, rtol=1e-12, atol=1e-14)


def test_max_group_one_head_per_group_is_the_sum():
    rng = np.random.default_rng(11)
    q, k = _rand_qk(rng, 2, 5, 3, 3, 8, 23)
    np.testing.assert_allclose(O.attention_score_max_group(q, k)[0], O.attention_mass(q, k)[0],
                               rtol=1e-13)


def test_max_group_identical_heads_closed_form():
    """Heads of a group that share their queries see the same weights: max = sum / G."""
    rng = np.random.default_rng(12)
    nl, w, hkv, g, d, n = 2, 4, 2, 4, 8, 19
    base = O.bf16_round(rng.standard_normal((nl, w, hkv, d)))
    q = np.repeat(base, g, axis=2)                                       # [L][W][Hq][D]
    k = O.bf16_round(rng.standard_normal((nl, n, hkv, d)))
    np.testing.assert_allclose(O.attention_score_max_group(q, k)[0], O.attention_mass(q, k)[0] / g,
                               rtol=1e-13)


def test_max_group_bounds_and_totals():
    """max <= sum <= G * max per key; every softmax row sums to 1, so the total score
    lies between L*Hkv*W and L*Hq*W."""
    rng = np.random.default_rng(13)
    nl, w, hq, hkv, d, n = 2, 6, 8, 2, 16, 40
    q, k = _rand_qk(rng, nl, w, hq, hkv, d, n)
    smax, _ = O.attention_score_max_group(q, k)
    ssum, _ = O.attention_mass(q, k)
    assert (smax <= ssum * (1 + 1e-12)).all() and (ssum <= 4 * smax * (1 + 1e-12)).all()
    assert nl * hkv * w - 1e-9 <= smax.sum() <= nl * hq * w + 1e-9


def test_supplied_lse_closed_forms():
    """A supplied LSE equal to the true one changes nothing; shifting it by delta scales
    every recovered weight by exp(-delta) (ActKV Sec. 7.1: A = exp(s - LSE))."""
    rng = np.random.default_rng(14)
    q, k = _rand_qk(rng, 2, 3, 8, 2, 8, 15)
    for fn in (O.attention_mass, O.attention_score_max_group):
        s0, lse = fn(q, k)
        s1, _ = fn(q, k, lse=lse)
        np.testing.assert_allclose(s1, s0, rtol=1e-14)
        s2, _ = fn(q, k, lse=lse + 0.75)
        np.testing.assert_allclose(s2, s0 * math.exp(-0.75), rtol=1e-13)


# ---------------------------------------------------------------------------------------
# O2 MemDecay / H2O closed forms
# ---------------------------------------------------------------------------------------

def test_memdecay_idle_steps_closed_form():
    rng = np.random.default_rng(10)
    n = 50
    region = rng.integers(0, 7, n)
    b = rng.uniform(0, 2, 7)
    lam = rng.uniform(0.004, 0.05, 7)
    a0 = rng.uniform(0, 0.1, n)
    c0 = rng.integers(0, 100, n)
    rho, alpha, dt = 0.9, 1.3, 3
    a, c = a0.copy(), c0.copy()
    for _ in range(7):
        a, c, s = O.memdecay_update(np.zeros(n), region, b, lam, rho, alpha, 0.01, dt, a, c)
    np.testing.assert_allclose(a, rho ** 7 * a0, rtol=1e-13)
    assert (c == c0 + 7 * dt).all()
    np.testing.assert_allclose(s, b[region] * np.exp(-lam[region] * (c0 + 7 * dt))
                               + alpha * rho ** 7 * a0, rtol=1e-13)


def test_memdecay_constant_attention_fixed_point():
    n = 5
    region = np.arange(n)
    b = np.linspace(0.2, 1.8, 7)
    lam = np.full(7, 0.02)
    cval = 0.3
    a0 = np.array([0.0, 0.1, 0.5, 1.0, 2.0])
    a, c = a0.copy(), np.full(n, 40)
    rho = 0.8
    for step in range(1, 30):
        a, c, s = O.memdecay_update(np.full(n, cval), region, b, lam, rho, 2.0, 0.01, 1, a, c)
        np.testing.assert_allclose(a, cval + rho ** step * (a0 - cval), rtol=1e-12)
        assert (c == 0).all()
    np.testing.assert_allclose(s, b[region] + 2.0 * (cval + rho ** 29 * (a0 - cval)), rtol=1e-12)


def test_memdecay_half_life():
    """t_1/2 = ln 2 / lambda: after one half-life the decay term is b/2 (MemDecay)."""
    lam = math.log(2) / 64
    _, _, s = O.memdecay_update(np.zeros(1), [0], [1.7] + [0] * 6, [lam] + [0] * 6,
                                0.9, 0.0, 0.01, 64, np.zeros(1), np.zeros(1, dtype=np.int64))
    assert abs(s[0] - 0.85) < 1e-15
    gd = read_golden("memdecay_halflife.txt")
    # the generator's lambda range spans the measured half-lives (system .. scratchpad)
    lo, hi = 0.004, 0.05
    assert math.log(2) / hi <= gd["scratchpad_halflife"][0]
    assert math.log(2) / lo >= gd["system_halflife"][0]


def test_memdecay_reset_is_strict_and_zero_clock():
    tau = 0.01
    abar = np.array([tau, np.nextafter(tau, 1), 0.0])
    a, c, s = O.memdecay_update(abar, [1, 1, 1], [0, 0.5] + [0] * 5, [0, 0.1] + [0] * 5,
                                0.5, 1.0, tau, 2, np.zeros(3), np.array([10, 10, 10]))
    assert list(c) == [12, 0, 12]
    # dt = 0 gives s = b + alpha * a
    assert abs(s[1] - (0.5 + a[1])) < 1e-15


def test_h2o_accumulates():
    rng = np.random.default_rng(11)
    masses = [rng.uniform(0, 3, 9) for _ in range(4)]
    acc = np.zeros(9)
    for m in masses:
        acc, s = O.h2o_update(m, acc)
    np.testing.assert_allclose(acc, np.sum(masses, axis=0), rtol=1e-14)
    _, s2 = O.h2o_update(np.zeros(9), acc, bonus=np.full(9, 2.0))
    np.testing.assert_allclose(s2, acc + 2.0)


# ---------------------------------------------------------------------------------------
# O3 foresight: the bonus of each token, and the properties the pages fix for the
# per-span values (drawn by the input generator, as the planner would supply them)
# ---------------------------------------------------------------------------------------

def test_generated_span_bonus_has_the_pages_properties():
    """PACE fixes three properties of the planner's bonus: a constant floor of 50K, the
    soonest-needed span first, and dominance over the unprotected attention scores it
    measured.  The generator's stand-in must have all three."""
    gd = read_golden("pace_numbers.txt")
    floor = gd["foresight_floor"]
    w = synth.workload("qwen3-8b-n100k", n_tokens=50000, n_spans=400)
    sid, bonus = synth.spans(w, seed=5, n_steps=16, p_needed=0.5, floor=floor)
    assert bonus.dtype == torch.float32 and bonus.shape == (400,)
    assert sid.min() == 0 and sid.max() == 399 and bool((sid[1:] >= sid[:-1]).all())
    b = bonus.double().numpy()
    needed = b > 0
    assert 50 < needed.sum() < 350
    assert b[needed].min() >= floor and b[needed].max() <= 2 * floor
    unprot = np.array([gd["max_unprotected_1m"], gd["max_unprotected_2m"]])
    assert b[needed].min() > unprot.max()
    # soonest first: the distinct values, ordered, are floor*(1+1/d) for d = 1, 2, ...
    vals = np.unique(b[needed])[::-1]
    d = floor / (vals - floor)
    np.testing.assert_allclose(d, np.rint(d), rtol=0, atol=1e-3)
    assert (np.diff(np.rint(d)) > 0).all() and np.rint(d).max() <= 16


def test_token_bonus_by_hand():
    """A token takes its span's bonus; id -1 (no span) and ids that name no span of the
    table get none."""
    bonus = np.array([10.0, 20.0, 30.0])
    sid = np.array([-1, 0, 2, 3, 1, -7, 2 ** 31 - 1, 0])
    assert O.token_bonus(sid, bonus).tolist() == [0.0, 10.0, 30.0, 0.0, 20.0, 0.0, 0.0, 10.0]
    # through the score step: H2O adds exactly that bonus to the accumulated mass
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 2, 8))
    k = rng.standard_normal((1, 8, 1, 8))
    out = O.score_step(q, k, policy="h2o", span_id=sid, span_bonus=bonus)
    want = [0.0, 10.0, 30.0, 0.0, 20.0, 0.0, 0.0, 10.0]
    np.testing.assert_allclose(out["token_score"] - out["accum"], want, rtol=0, atol=1e-9)
    # and MemDecay adds it on top of the decay and EWMA terms
    md = dict(region=np.zeros(8, np.uint8), base_prio=[1.0], decay_rate=[0.5],
              ewma=np.full(8, 0.25), clock=np.arange(8))
    out = O.score_step(q, k, policy="memdecay", span_id=sid, span_bonus=bonus, **md)
    plain = O.score_step(q, k, policy="memdecay", **md)
    np.testing.assert_allclose(out["token_score"] - plain["token_score"], want, rtol=0,
                               atol=1e-9)


def test_region_labels_outside_the_table():
    """A label at or above the number of regions names no region: no base priority, no
    decay, no region pinning."""
    a, c, s = O.memdecay_update(np.array([0.0, 0.0]), np.array([1, 9]), [1.0, 2.0], [0.1, 0.1],
                                rho=0.5, alpha=1.0, tau=0.01, dt_steps=1, ewma=[0.5, 0.5],
                                clock=[0, 0])
    assert c.tolist() == [1, 1]
    np.testing.assert_allclose(s, [2.0 * math.exp(-0.1) + 0.25, 0.25], rtol=1e-15)
    pin = O.pinned_tokens(4, np.array([0, 3, 7, 40]), pinned_regions=(1 << 3) | (1 << 7) | 1,
                          n_regions=5)
    assert pin.tolist() == [True, True, False, False]


# ---------------------------------------------------------------------------------------
# pins / page aggregation
# ---------------------------------------------------------------------------------------

def test_pinned_rules_and_pages():
    n = 37
    region = np.array([0] * 5 + [3] * 20 + [5] * 12)
    pin = O.pinned_tokens(n, region, pinned_regions=(1 << 0) | (1 << 5), n_sink=2, n_recent=3)
    assert pin[:5].all() and not pin[5:25].any() and pin[25:].all()
    pin2 = O.pinned_tokens(n, region, 0, n_sink=4, n_recent=2)
    assert list(np.nonzero(pin2)[0]) == [0, 1, 2, 3, 35, 36]
    s = np.arange(n, dtype=np.float64)
    pm = O.page_mean(s, 16)
    full = s[:32].reshape(2, 16).mean(axis=1)
    np.testing.assert_allclose(pm[:2], full)
    assert pm[2] == np.mean([32, 33, 34, 35, 36])
    assert list(O.page_any(pin2, 16)) == [True, False, True]


# ---------------------------------------------------------------------------------------
# O4 selection
# ---------------------------------------------------------------------------------------

def _valid_by_definition(score, pinned, budget, kept):
    """Characterisation: kept contains every pinned item, has size min(max(B,#pin), n),
    and every kept unpinned item precedes every evicted unpinned item in the order
    (score desc, index asc)."""
    n = len(score)
    kept = set(kept)
    npin = int(sum(pinned))
    if not all(i in kept for i in range(n) if pinned[i]):
        return False
    if len(kept) != min(n, max(budget, npin)):
        return False
    for i in kept:
        if pinned[i]:
            continue
        for e in range(n):
            if e in kept or pinned[e]:
                continue
            if not (score[i] > score[e] or (score[i] == score[e] and i < e)):
                return False
    return True


def test_select_exhaustive_brute_force():
    alphabet = [0.0, 0.5, 1.0]
    count = 0
    for n in range(1, 6):
        for scores in itertools.product(alphabet, repeat=n):
            for pmask in range(0, 1 << n, 3):
                pinned = [(pmask >> i) & 1 for i in range(n)]
                for budget in range(0, n + 1):
                    kept, status = O.select_items(np.array(scores), np.array(pinned), budget)
                    # exactly one subset satisfies the characterisation
                    valid = [c for size in range(n + 1)
                             for c in itertools.combinations(range(n), size)
                             if _valid_by_definition(scores, pinned, budget, c)]
                    assert len(valid) == 1
                    assert list(kept) == list(valid[0])
                    assert bool(status & O.STATUS_PINNED_OVER_BUDGET) == (sum(pinned) > budget)
                    count += 1
    assert count > 1000


def _before(score, i, e):
    """Item i precedes item e in the selection order: numbers before NaN, higher score
    first, -0 equal to +0, the lower index first on a tie."""
    ki = (1, 0.0) if math.isnan(score[i]) else (0, -(score[i] + 0.0))
    ke = (1, 0.0) if math.isnan(score[e]) else (0, -(score[e] + 0.0))
    return (ki, i) < (ke, e)


@hyp.settings(max_examples=400, deadline=None)
@hyp.given(st.data())
def test_select_total_order_brute_force(data):
    """Every float class (NaN, infinities, signed zeros, ties) against the brute-force
    characterisation: the kept set holds every pinned item, has min(n, max(B, #pinned))
    items, and each kept unpinned item precedes each evicted unpinned one."""
    vals = [math.nan, -math.inf, -1.0, -0.0, 0.0, 0.5, 1.0, math.inf]
    score = data.draw(st.lists(st.sampled_from(vals), min_size=1, max_size=7))
    n = len(score)
    pinned = data.draw(st.lists(st.booleans(), min_size=n, max_size=n))
    budget = data.draw(st.integers(0, n + 1))
    kept, status = O.select_items(np.array(score), np.array(pinned), budget)
    npin = sum(pinned)
    want = None
    for size in range(n + 1):
        for c in itertools.combinations(range(n), size):
            cs = set(c)
            if not all(i in cs for i in range(n) if pinned[i]) or size != min(n, max(budget, npin)):
                continue
            if all(_before(score, i, e) for i in cs if not pinned[i]
                   for e in range(n) if e not in cs and not pinned[e]):
                assert want is None, "the characterisation admits one set only"
                want = list(c)
    assert list(kept) == want
    assert bool(status & O.STATUS_NAN_SCORE) == any(math.isnan(v) for v in score)
    assert bool(status & O.STATUS_PINNED_OVER_BUDGET) == (npin > budget)


def test_select_properties_random():
    for seed in range(5):
        s = synth.scores(3000, seed=seed, alphabet=[0.1, 0.2, 0.3, 0.4] if seed % 2 else None)
        pin = synth.pinned_mask(3000, seed=seed, frac=0.02).numpy().astype(bool)
        budget = 500
        kept, _ = O.select_items(s.double().numpy(), pin, budget)
        assert len(kept) == budget
        assert (np.diff(kept) > 0).all()
        assert set(np.nonzero(pin)[0]) <= set(kept)
        sv = s.double().numpy()
        ev = np.setdiff1d(np.arange(3000), kept)
        ev = ev[~pin[ev]]
        kn = kept[~pin[kept]]
        assert sv[kn].min() >= sv[ev].max()


def test_select_nan_last_and_signed_zero():
    s = np.array([np.nan, -0.0, 0.0, -1.0, np.nan, 2.0])
    kept, status = O.select_items(s, None, 3)
    assert list(kept) == [1, 2, 5] and status & O.STATUS_NAN_SCORE
    kept, _ = O.select_items(s, None, 5)
    assert list(kept) == [0, 1, 2, 3, 5]


def test_expand_pages_partial_tail():
    assert list(O.expand_items([0, 2], 4, 10)) == [0, 1, 2, 3, 8, 9]


# ---------------------------------------------------------------------------------------
# O5 Penelope
# ---------------------------------------------------------------------------------------

def test_penelope_illustrative_example():
    gd = read_golden("penelope_cost.txt")
    u = gd["linear_units"]
    p, priv, free = gd["example_prefix"], gd["example_private"], gd["example_free"]
    end = O.recompute_cost(p + priv - free, p + priv, u)
    front = O.recompute_cost(p, p + free, u)
    ratio = end / front
    assert abs(ratio - gd["example_ratio_about"]) < 0.05
    assert abs(ratio - 124551.5 / 54551.5) < 1e-12
    # mean tokens-before of each choice, as the page states
    assert abs((end / free - u) - gd["example_end_mean_before"]) < 1000
    assert abs((front / free - u) - gd["example_front_mean_before"]) < 1000


@pytest.mark.parametrize("ctx_k,key", [(8, "measure_8k_speedup"), (128, "measure_128k_speedup")])
@pytest.mark.parametrize("with_append", [False, True])
def test_penelope_measurement_within_4pct(ctx_k, key, with_append):
    gd = read_golden("penelope_cost.txt")
    u = gd["linear_units"]
    n = ctx_k * 1024
    e = int(round(gd["measure_frac"] * n))
    start = gd["measure_start"]
    add = O.recompute_cost(n, n + gd["measure_append"], u) if with_append else 0.0
    end = O.recompute_cost(n - e, n, u) + add
    front = O.recompute_cost(start, start + e, u) + add
    assert abs(end / front / gd[key] - 1) < gd["measure_tolerance"]


def test_penelope_segment_blocks():
    assert O.segment_evict_len(131072, 16384, 39322, 16) == 39328
    keep = O.select_segment(100, 10, 7, 4)
    assert list(keep) == list(range(10)) + list(range(18, 100))
    assert O.segment_evict_len(40, 30, 50, 16) == 10


# ---------------------------------------------------------------------------------------
# O4b ActKV LRFU and top-p hit mask (Sec. 5.1, Algorithm 1)
# ---------------------------------------------------------------------------------------

def _rank_order(sc):
    key = np.where(np.isnan(sc), -np.inf, sc.astype(np.float64))
    key = np.where(key == 0, 0.0, key)
    return sorted(range(len(sc)), key=lambda j: (-key[j], j))


def _exact_weights(sc):
    """Each finite positive float32 score as an exact rational, else 0 (independent of the
    oracle's integer scaling)."""
    return [Fraction(float(x)) if math.isfinite(float(x)) and float(x) > 0 else Fraction(0)
            for x in np.asarray(sc, np.float32)]


def _hits_by_definition(sc, p):
    """Per-entry form of the top-p set: an entry with weight is a hit exactly when the
    weight of the entries ranked before it has not yet reached p times the total."""
    w = _exact_weights(sc)
    target = Fraction(float(np.float32(p))) * sum(w)
    order = _rank_order(np.asarray(sc, np.float32))
    before = {}
    acc = Fraction(0)
    for j in order:
        before[j] = acc
        acc += w[j]
    return np.array([w[j] > 0 and before[j] < target for j in range(len(w))])


@pytest.mark.parametrize("seed", range(8))
def test_topp_hit_mask_is_the_minimal_prefix(seed):
    """The hits reach p times the total exactly, dropping the lowest-ranked hit falls short
    of it, and every hit ranks above every positive-weight miss (total order: score
    descending, index ascending)."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 40))
    sc = rng.choice([0.0, -0.0, 0.25, 0.5, 1e-3, 3.0, 1e-40, float(rng.random())], n).astype(np.float32)
    if seed % 3 == 0:
        sc[rng.integers(0, n)] = np.nan
    p = float(rng.choice([0.5, 0.9, 0.999, 1.0]))
    hit = O.topp_hit_mask(sc, p)
    w = _exact_weights(sc)
    target = Fraction(float(np.float32(p))) * sum(w)
    hw = [w[j] for j in range(n) if hit[j]]
    if target == 0:
        assert not hit.any()
        return
    assert sum(hw) >= target
    ranks = {j: r for r, j in enumerate(_rank_order(sc))}
    last = max((j for j in range(n) if hit[j]), key=lambda j: ranks[j])
    assert sum(hw) - w[last] < target
    for j in range(n):
        if not hit[j] and w[j] > 0:
            assert all(ranks[h] < ranks[j] for h in range(n) if hit[h])
    assert all(w[j] > 0 for j in range(n) if hit[j])


def test_topp_exhaustive_against_the_per_entry_definition():
    """Every score vector of length <= 5 over an alphabet with ties, zeros, a negative, a
    subnormal and NaN, at several p: the oracle's prefix walk equals the per-entry form."""
    alphabet = [0.5, 0.25, 0.0, -1.0, 1e-40, float("nan")]
    ps = [0.0, 0.25, 0.5, 0.75, float(np.nextafter(np.float32(0.5), np.float32(1))), 1.0]
    count = 0
    for n in range(1, 6):
        for combo in itertools.product(alphabet, repeat=n):
            sc = np.array(combo, dtype=np.float32)
            for p in ps:
                assert (O.topp_hit_mask(sc, p) == _hits_by_definition(sc, p)).all(), (combo, p)
                count += 1
    assert count > 50_000


def test_topp_random_against_the_per_entry_definition():
    rng = np.random.default_rng(77)
    for _ in range(40):
        n = int(rng.integers(1, 300))
        sc = (rng.random(n) ** rng.integers(1, 30)).astype(np.float32)
        sc[rng.random(n) < 0.1] = 0.0
        p = float(rng.choice([0.1, 0.5, 0.9, 0.99, 1.0, float(rng.random())]))
        assert (O.topp_hit_mask(sc, p) == _hits_by_definition(sc, p)).all()


def test_exact_score_units():
    vals = np.array([1.0, 0.1, 3.4028235e38, 1.1754944e-38, 1e-45, 1e-40, 0.0, -0.0, -2.0,
                     np.inf, np.nan], dtype=np.float32)
    u = O.exact_score_units(vals)
    for x, got in zip(vals, u):
        want = Fraction(float(x)) * 2 ** 149 if np.isfinite(x) and x > 0 else 0
        assert got == want and int(want) == want
    assert u[4] == 1                                   # the smallest subnormal is one unit


def test_topp_special_cases():
    # one entry holding 95% of the weight is the only hit at p = 90%
    sc = np.array([0.01] * 5 + [0.95], dtype=np.float32)
    assert O.topp_hit_mask(sc, 0.9).tolist() == [False] * 5 + [True]
    # p = 1 takes every entry with weight; equal scores are taken by index
    sc = np.array([0.2, 0.2, 0.2, 0.0, 0.2, 0.2], dtype=np.float32)
    assert O.topp_hit_mask(sc, 1.0).tolist() == [True, True, True, False, True, True]
    assert O.topp_hit_mask(sc, 0.5).tolist() == [True, True, True, False, False, False]
    assert not O.topp_hit_mask(np.zeros(7, np.float32), 0.9).any()
    assert not O.topp_hit_mask(sc, 0.0).any()
    # an exact boundary: 0.5 of a total of 1 is reached by the first entry alone; the next
    # float32 above 0.5 needs the second one too
    sc = np.array([0.25, 0.5, 0.25], dtype=np.float32)
    assert O.topp_hit_mask(sc, 0.5).tolist() == [False, True, False]
    up = float(np.nextafter(np.float32(0.5), np.float32(1)))
    assert O.topp_hit_mask(sc, up).tolist() == [True, True, False]
    # p is the float32 the device receives: float32(0.9) * (0.9f + 0.1f) is below 0.9f, so
    # the first entry alone reaches it, while the decimal 0.9 would need both
    sc = np.array([0.9, 0.1], dtype=np.float32)
    t = Fraction(float(sc[0])) + Fraction(float(sc[1]))
    assert Fraction(float(np.float32(0.9))) * t <= Fraction(float(sc[0])) < Fraction(0.9) * t
    assert O.topp_hit_mask(sc, 0.9).tolist() == [True, False]


def test_topp_every_positive_score_is_a_hit_at_p_one():
    """At p = 1 the set must cover the whole weight, so every positive score is a hit,
    however small next to the others (scores from 1e-45 to 1)."""
    rng = np.random.default_rng(12)
    sc = np.float32(10.0) ** rng.uniform(-45, 0, 5000).astype(np.float32)
    sc = sc.astype(np.float32)
    sc[:50] = 0.0
    assert (sc[50:] > 0).all() and sc.min() == 0 and (sc[50:] < 1e-38).any()
    hit = O.topp_hit_mask(sc, 1.0)
    assert (hit == (sc > 0)).all()
    # just below p = 1 the smallest scores stay out: together they weigh less than the
    # missing 2**-24 of the total
    below = O.topp_hit_mask(sc, float(np.nextafter(np.float32(1), np.float32(0))))
    assert below.sum() < hit.sum() and below[np.argmax(sc)]


def test_lrfu_update_rule():
    """KS <- lambda KS + AttnScore on hits, lambda KS on misses (Algorithm 1, its keep-score update):
    lambda = 0 keeps only the current hits, lambda = 1 accumulates, and a missed entry
    decays geometrically instead of dropping out."""
    a = np.array([0.5, 0.25, 0.125, 0.125], dtype=np.float32)  # 0.75 < 0.85 <= 0.875
    ks0 = np.array([1.0, 2.0, 3.0, 4.0])
    ks, hit = O.lrfu_update(ks0, a, p=0.85, decay=0.0)
    assert hit.tolist() == [True, True, True, False]
    np.testing.assert_allclose(ks, np.where(hit, a.astype(np.float64), 0.0))
    ks, _ = O.lrfu_update(ks0, a, p=1.0, decay=1.0)
    np.testing.assert_allclose(ks, ks0 + a.astype(np.float64))
    ks = np.array([1.0, 0.0])
    for _ in range(5):
        ks, hit = O.lrfu_update(ks, np.array([0.0, 1.0], np.float32), p=0.9, decay=0.5)
        assert hit.tolist() == [False, True]
    assert ks[0] == 0.5 ** 5 and ks[1] == 1.0 + 0.5 + 0.25 + 0.125 + 0.0625


# ---------------------------------------------------------------------------------------
# O4c ActKV in-place tail compaction (Sec. 7.2, Algorithm 4)
# ---------------------------------------------------------------------------------------

def test_tail_compaction_worked_example():
    """40 used slots in blocks of 8 and a budget of 12: Y = 5, X = 2, region [24, 36).
    Kept 33 and 35 stay; 1, 5, 20 and 38 move into the first free slots 24..27."""
    start, end, src, dst, over = O.tail_compaction_pairs(40, [1, 5, 20, 33, 35, 38], 12, 8)
    assert (start, end, over) == (24, 36, False)
    assert src.tolist() == [1, 5, 20, 38] and dst.tolist() == [24, 25, 26, 27]
    arr = np.arange(48)[None, :] * 10
    out = O.tail_compact(arr, src, dst)
    assert out[0, 24:28].tolist() == [10, 50, 200, 380] and out[0, 33] == 330 and out[0, 35] == 350
    assert (out[0, :24] == arr[0, :24]).all()
    # more kept entries than the region holds: only the first ones are paired
    *_, src2, dst2, over2 = O.tail_compaction_pairs(40, list(range(0, 40, 3)), 12, 8)
    assert over2 and len(src2) == len(dst2)


@pytest.mark.parametrize("seed", range(6))
def test_tail_compaction_invariants(seed):
    rng = np.random.default_rng(320 + seed)
    bs = int(rng.choice([4, 16, 64]))
    n = int(rng.integers(bs + 1, 600))
    budget = int(rng.integers(1, n))
    n_keep = int(rng.integers(0, budget + 1))
    keep = np.sort(rng.choice(n, n_keep, replace=False))
    start, end, src, dst, over = O.tail_compaction_pairs(n, keep, budget, bs)
    y, x = -(-n // bs), -(-budget // bs)
    assert start == (y - x) * bs and end - start == budget and end <= y * bs
    assert not over
    window = set(range(start, end))
    assert set(dst.tolist()) <= window and not (set(dst.tolist()) & set(keep.tolist()))
    assert not (set(src.tolist()) & window) and len(set(src.tolist()) | set(dst.tolist())) == 2 * len(src)
    data = rng.standard_normal((2, y * bs))
    out = O.tail_compact(data, src, dst)
    # every kept entry now lives inside the region, each exactly once
    placed = [out[:, j] for j in sorted((set(keep.tolist()) & window) | set(dst.tolist()))]
    assert len(placed) == n_keep
    got = sorted(tuple(c) for c in placed)
    want = sorted(tuple(c) for c in data[:, keep].T)
    assert got == want


# ---------------------------------------------------------------------------------------
# O6 re-rotation (PACE Sec. 3.2, Proposition 1)
# ---------------------------------------------------------------------------------------

def _rope_hf(x, pos, theta):
    """Model-side rotary embedding written the Hugging Face way (rotate_half)."""
    x = torch.from_numpy(np.asarray(x, dtype=np.float64))
    d = x.shape[-1]
    inv = 1.0 / (theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    freqs = torch.as_tensor(pos, dtype=torch.float64)[..., None] * inv
    emb = torch.cat([freqs, freqs], dim=-1)
    rot = torch.cat([-x[..., d // 2:], x[..., : d // 2]], dim=-1)
    return (x * emb.cos() + rot * emb.sin()).numpy()


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_proposition1_exact_rerotation(theta):
    rng = np.random.default_rng(12)
    k0 = rng.standard_normal((20, 128))
    p = rng.integers(0, 1_000_000, 20)
    qn = rng.integers(0, 8192, 20)
    cached = _rope_hf(k0, p, theta)
    re = O.rope_rotate(cached, qn - p, theta)
    want = _rope_hf(k0, qn, theta)
    np.testing.assert_allclose(re, want, atol=1e-9)


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((5, 128))
    delta = np.array([1, -3, 1000, -39328, 77777])
    out = O.rope_rotate(k, delta, 1e6)
    z = k[:, :64] + 1j * k[:, 64:]
    inv = np.power(1e6, -np.arange(64) * 2.0 / 128)
    zr = z * np.exp(1j * delta[:, None] * inv)
    np.testing.assert_allclose(out[:, :64], zr.real, atol=1e-12)
    np.testing.assert_allclose(out[:, 64:], zr.imag, atol=1e-12)


def test_rotation_composition_shift_invariance_norms():
    rng = np.random.default_rng(14)
    x, y = rng.standard_normal((2, 128))
    a, b, s = 1234, 99, 50_000
    r1 = O.rope_rotate(O.rope_rotate(x, a, 1e6), b - a, 1e6)
    np.testing.assert_allclose(r1, O.rope_rotate(x, b, 1e6), atol=1e-11)
    d1 = O.rope_rotate(x, a, 1e6) @ O.rope_rotate(y, b, 1e6)
    d2 = O.rope_rotate(x, a + s, 1e6) @ O.rope_rotate(y, b + s, 1e6)
    assert abs(d1 - d2) < 1e-10
    rx = O.rope_rotate(x, 777, 1e6)
    np.testing.assert_allclose(rx[:64] ** 2 + rx[64:] ** 2, x[:64] ** 2 + x[64:] ** 2, rtol=1e-12)


def test_compact_rerope_definition():
    rng = np.random.default_rng(15)
    nl, n, hk, d = 2, 30, 2, 128
    k = O.bf16_round(rng.standard_normal((nl, n, hk, d)))
    v = O.bf16_round(rng.standard_normal((nl, n, hk, d)))
    keep = np.array([0, 1, 2, 7, 8, 20, 29])
    old_pos = np.arange(n) + 100
    old_pos[:3] = [0, 1, 2]                       # first three keep their place: delta 0
    k2, v2, newp = O.compact_rerope(k, v, keep, old_pos, 0, 1e6)
    assert list(newp) == list(range(len(keep)))
    assert (v2 == v[:, keep]).all()
    assert (k2[:, :3] == k[:, :3]).all()          # delta 0: verbatim
    for r, j in enumerate(keep):
        want = O.bf16_round(O.rope_rotate(k[:, j], r - old_pos[j], 1e6))
        assert (k2[:, r] == want).all()
    # two roundings at most through bf16 storage: round-trip to a far position and back
    k_far = O.bf16_round(O.rope_rotate(k[:, 5], 100_000, 1e6))
    back = O.bf16_round(O.rope_rotate(k_far, -100_000, 1e6))
    # bf16 keeps 8 significant bits: each RNE rounding moves a component by at most
    # 2^-8 of its magnitude, hence a pair by at most 2^-8 of its norm; rotation preserves
    # the norm, so two roundings stay within 2^-8 * (2 + 2^-8) of it
    x, y = k[:, 5, :, :64], k[:, 5, :, 64:]
    norm = np.sqrt(x ** 2 + y ** 2)
    err = np.sqrt((back[..., :64] - x) ** 2 + (back[..., 64:] - y) ** 2)
    assert (err <= 2 ** -8 * (2 + 2 ** -8) * norm + 1e-30).all()
    # no renumbering keeps positions and every key
    k3, _, p3 = O.compact_rerope(k, v, keep, old_pos, -1, 1e6)
    assert (p3 == old_pos[keep]).all() and (k3 == k[:, keep]).all()


def test_scaled_inv_freq_special_cases():
    """PACE Sec. 3.5's static scalings against their defining cases: linear divides every
    frequency; with factor 1 Llama-3 and YaRN reduce to plain RoPE; Llama-3 keeps the
    high-frequency dims, divides the low-frequency ones and blends in between; YaRN keeps
    dims turning more than beta_fast times over the original context and divides those
    turning less than beta_slow times."""
    base = 5e5
    d = O.scaled_inv_freq("default", base)
    np.testing.assert_array_equal(d, np.power(base, -np.arange(64) / 64.0))
    np.testing.assert_allclose(O.scaled_inv_freq("linear", base, factor=4.0), d / 4.0, rtol=1e-15)
    np.testing.assert_allclose(O.scaled_inv_freq("llama3", base, factor=1.0), d, rtol=1e-15)
    np.testing.assert_allclose(O.scaled_inv_freq("yarn", base, factor=1.0), d, rtol=1e-15)
    wl = 2 * math.pi / d
    ll = O.scaled_inv_freq("llama3", base, factor=8.0, original_max_position=8192,
                           low_freq_factor=1.0, high_freq_factor=4.0)
    hi, lo = wl < 8192 / 4.0, wl > 8192 / 1.0
    assert hi.any() and lo.any() and (~hi & ~lo).any()
    np.testing.assert_array_equal(ll[hi], d[hi])
    np.testing.assert_allclose(ll[lo], d[lo] / 8.0, rtol=1e-15)
    mid = ~hi & ~lo
    assert ((ll[mid] > d[mid] / 8.0) & (ll[mid] < d[mid])).all()
    assert (np.diff(ll) < 0).all()
    r = 4096 / wl
    fast, slow = r > 32.0, r < 1.0
    assert fast.any() and slow.any()
    for kind in ("yarn", "yarn_ratio"):
        np.testing.assert_allclose(O.scaled_inv_freq(kind, base, factor=1.0), d, rtol=1e-15)
        ya = O.scaled_inv_freq(kind, base, factor=16.0, original_max_position=4096)
        np.testing.assert_allclose(ya[fast], d[fast], rtol=1e-15)
        np.testing.assert_allclose(ya[slow], d[slow] / 16.0, rtol=1e-15)
        m = ~fast & ~slow
        assert ((ya[m] >= d[m] / 16.0) & (ya[m] <= d[m])).all()
        assert (np.diff(ya) < 0).all()
    # the pair turning exactly beta times over L sits at D ln(L / (2 pi beta)) / (2 ln base)
    i32 = 128 * math.log(4096 / (2 * math.pi * 32.0)) / (2 * math.log(base))
    assert abs(4096 / (2 * math.pi / base ** (-2 * i32 / 128)) - 32.0) < 1e-9


def _hf_table(kind, base, factor, L, **params):
    """The frequencies transformers' model code rotates with (it builds them in float32)."""
    from transformers import PretrainedConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    rp = dict(rope_type=kind, rope_theta=base, factor=factor, original_max_position_embeddings=L, **params)
    cfg = PretrainedConfig(hidden_size=4096, num_attention_heads=32, head_dim=128,
                           max_position_embeddings=int(L * factor), rope_parameters=rp)
    inv, _ = ROPE_INIT_FUNCTIONS[kind](cfg, "cpu")
    return inv.double().numpy()


@pytest.mark.parametrize("base,factor,L", [(1e6, 4.0, 32768), (5e5, 8.0, 8192), (1e4, 16.0, 4096),
                                           (150000.0, 32.0, 4096), (1e6, 2.0, 131072)])
def test_scaled_tables_match_transformers(base, factor, L):
    """Llama-3 and YaRN tables against the ones transformers' model code caches keys with
    (an independent implementation).  Its tables are float32, so the bar is a few float32
    roundings (4e-6 relative).  The YaRN paper's ratio form differs inside the band."""
    pytest.importorskip("transformers")
    ll = _hf_table("llama3", base, factor, L, low_freq_factor=1.0, high_freq_factor=4.0)
    np.testing.assert_allclose(O.scaled_inv_freq("llama3", base, factor=factor, original_max_position=L),
                               ll, rtol=4e-6, atol=0)
    for params in (dict(beta_fast=32.0, beta_slow=1.0), dict(beta_fast=16.0, beta_slow=2.0, truncate=False)):
        hf = _hf_table("yarn", base, factor, L, **params)
        ours = O.scaled_inv_freq("yarn", base, factor=factor, original_max_position=L, **params)
        np.testing.assert_allclose(ours, hf, rtol=4e-6, atol=0)
    ratio = O.scaled_inv_freq("yarn_ratio", base, factor=factor, original_max_position=L)
    assert np.abs(ratio / _hf_table("yarn", base, factor, L) - 1).max() > 1e-2


@pytest.mark.parametrize("kind", ["linear", "llama3", "yarn", "yarn_ratio"])
def test_proposition1_holds_for_scaled_tables(kind):
    """Re-rotating a key cached at p by q - p gives the key cached at q for any fixed
    frequency table (the model-side rotation written the rotate_half way)."""
    inv = O.scaled_inv_freq(kind, 5e5, factor=8.0, original_max_position=8192)
    rng = np.random.default_rng(18)
    k0 = rng.standard_normal((10, 128))
    p, qn = rng.integers(0, 500_000, 10), rng.integers(0, 8192, 10)

    def hf(x, pos):
        f = torch.as_tensor(pos, dtype=torch.float64)[:, None] * torch.from_numpy(inv)
        emb = torch.cat([f, f], dim=-1)
        xt = torch.from_numpy(x)
        rot = torch.cat([-xt[:, 64:], xt[:, :64]], dim=-1)
        return (xt * emb.cos() + rot * emb.sin()).numpy()

    np.testing.assert_allclose(O.rope_rotate(hf(k0, p), qn - p, inv_freq=inv), hf(k0, qn), atol=1e-9)


def _pair_error(k, true):
    """Largest error of a rotation pair relative to the pair's norm."""
    e = np.sqrt((k[..., :64] - true[..., :64]) ** 2 + (k[..., 64:] - true[..., 64:]) ** 2)
    n = np.sqrt(true[..., :64] ** 2 + true[..., 64:] ** 2)
    return float((e / n).max())


def test_reference_store_error_stays_two_roundings():
    """PACE Sec. 3.2: deriving every position from the stored copy keeps the error at
    about two bf16 roundings however many renumbers a key survives, while re-rotating the
    stored key adds one rounding per position change."""
    rng = np.random.default_rng(19)
    nl, n, hk = 1, 48, 2
    inv = O.scaled_inv_freq("default", 1e6)
    x = rng.standard_normal((nl, n, hk, 128))                    # keys before rotation
    pos0 = rng.integers(0, 8192, n)
    k_store = O.bf16_round(O.rope_rotate(x, pos0[None, :, None], inv_freq=inv))
    k_plain = k_store.copy()
    v = np.zeros_like(k_store)
    ref_k, ref_pos = np.zeros_like(k_store), np.full(n, O.REF_NONE)
    keep = np.arange(n)
    pos_s, pos_p, prev = pos0, pos0, -1
    for step in range(60):
        base = int(rng.integers(0, 4096))
        base = base + 1 if base == prev else base
        prev = base
        k_store, _, pos_s, ref_k, ref_pos, used = O.compact_rerope_store(
            k_store, v, keep, pos_s, base, inv, ref_k, ref_pos)
        k_plain, _, pos_p = O.compact_rerope(k_plain, v, keep, pos_p, base, 1e6)
        assert used.all() == (step > 0)
        assert (ref_pos == pos0).all()                # the store keeps the cached copy
    assert (pos_s == pos_p).all()
    true = O.rope_rotate(x, pos_s[None, :, None], inv_freq=inv)
    bound = 2.0 ** -8 * (2 + 2.0 ** -8)                      # two roundings (see above)
    assert _pair_error(k_store, true) <= bound
    assert _pair_error(k_plain, true) > bound                # compounding without the store


def test_reference_store_first_use_and_foreign_entry():
    """With an empty store the keys equal plain compaction and moved keys are stored at
    their old positions; an entry that fails the check against the cached key (its slot
    was reused) is ignored and replaced."""
    rng = np.random.default_rng(20)
    nl, n, hk = 2, 24, 2
    k = O.bf16_round(rng.standard_normal((nl, n, hk, 128)))
    v = O.bf16_round(rng.standard_normal((nl, n, hk, 128)))
    old = np.arange(n) + 50
    old[:4] = np.arange(4)                                   # ranks 0..3 keep their place
    keep = np.array([0, 1, 2, 3, 9, 10, 17, 23])
    inv = O.scaled_inv_freq("default", 1e6)
    empty_k, empty_p = np.zeros_like(k), np.full(n, O.REF_NONE)
    k1, v1, p1, rk, rp, used = O.compact_rerope_store(k, v, keep, old, 0, inv, empty_k, empty_p)
    k0, v0, p0 = O.compact_rerope(k, v, keep, old, 0, 1e6)
    assert (k1 == k0).all() and (v1 == v0).all() and (p1 == p0).all() and not used.any()
    assert (rp[:4] == O.REF_NONE).all() and (rp[4:] == old[keep[4:]]).all()
    assert (rk[:, 4:] == k[:, keep[4:]]).all()
    # slot 9 holds a stale entry of another key: the check fails, the slot is re-seeded
    bad_k, bad_p = empty_k.copy(), empty_p.copy()
    bad_k[:, 9] = O.bf16_round(rng.standard_normal((nl, hk, 128)))
    bad_p[9] = 40
    k2, _, _, rk2, rp2, used2 = O.compact_rerope_store(k, v, keep, old, 0, inv, bad_k, bad_p)
    assert not used2.any() and (k2 == k0).all()
    assert rp2[4] == old[9] and (rk2[:, 4] == k[:, 9]).all()
    # a valid entry is used even when the cached key is not where it was stored
    good_k, good_p = empty_k.copy(), empty_p.copy()
    good_k[:, 17] = O.bf16_round(rng.standard_normal((nl, hk, 128)))
    good_p[17] = 5
    kc = k.copy()
    kc[:, 17] = O.bf16_round(O.rope_rotate(good_k[:, 17], old[17] - 5, inv_freq=inv))
    k3, _, _, rk3, rp3, used3 = O.compact_rerope_store(kc, v, keep, old, 0, inv, good_k, good_p)
    assert used3[6] and used3.sum() == 1 and rp3[6] == 5
    want = O.bf16_round(O.rope_rotate(good_k[:, 17], 6 - 5, inv_freq=inv))
    assert (k3[:, 6] == want).all()


def test_evicted_tokens_partition():
    assert O.evicted_tokens(10, [0, 3, 4, 9]).tolist() == [1, 2, 5, 6, 7, 8]
    rng = np.random.default_rng(21)
    for n in (1, 17, 1000):
        keep = np.sort(rng.choice(n, int(rng.integers(0, n + 1)), replace=False))
        ev = O.evicted_tokens(n, keep)
        assert len(ev) + len(keep) == n and not set(ev.tolist()) & set(keep.tolist())
        assert (np.diff(ev) > 0).all()
        # the e-th evicted token is e plus the kept tokens before it
        for e in range(0, len(ev), max(1, len(ev) // 7)):
            assert ev[e] == e + int((keep < ev[e]).sum())


def test_load_rows_is_the_inverse_of_evicted_gather():
    """Dropping rows (the keep list's complement, gathered in order) and loading them back
    into the slots they came from restores the row exactly; other slots stay untouched."""
    rng = np.random.default_rng(61)
    k = rng.standard_normal((3, 50, 2, 8))
    keep = np.sort(rng.choice(50, 17, replace=False))
    ev = O.evicted_tokens(50, keep)
    rows = k[:, ev]
    blank = np.where(np.isin(np.arange(50), keep)[None, :, None, None], k, 0.0)
    assert (O.load_rows(blank, ev, rows) == k).all()
    other = O.load_rows(k, [3, 9], rows[:, :2])
    assert (other[:, 3] == rows[:, 0]).all() and (other[:, 9] == rows[:, 1]).all()
    untouched = np.setdiff1d(np.arange(50), [3, 9])
    assert (other[:, untouched] == k[:, untouched]).all()


@pytest.mark.parametrize("count,chunk", [(1, 4), (4, 4), (10, 4), (9, 3), (7, 16)])
def test_chunked_swap_moves_both_segments(count, chunk):
    """The swap through the small buffer ends exactly where an unbounded exchange would:
    the GPU slots hold the incoming CPU rows, every outgoing row sits in the CPU row
    reported for it, no other CPU row holding data is overwritten, and swapping the other
    way with the reported buffer undoes it."""
    rng = np.random.default_rng(count * 31 + chunk)
    n, p = 40, count + chunk + 12
    gpu = rng.standard_normal((2, n, 1, 4))
    pool = rng.standard_normal((2, p, 1, 4))
    slots = rng.choice(n, count, replace=False)
    in_first, buf_first = 5, 5 + count + 3            # buffer after the incoming segment
    g2, p2, out_rows, nxt = O.chunked_swap(gpu, pool, slots, in_first, buf_first, chunk)
    assert (g2[:, slots] == pool[:, in_first:in_first + count]).all()
    assert (p2[:, out_rows] == gpu[:, slots]).all()
    others = np.setdiff1d(np.arange(n), slots)
    assert (g2[:, others] == gpu[:, others]).all()
    # CPU rows outside the incoming segment and the buffer keep their data
    used = set(range(in_first, in_first + count)) | set(range(buf_first, buf_first + min(chunk, count)))
    keep_rows = [r for r in range(p) if r not in used]
    assert (p2[:, keep_rows] == pool[:, keep_rows]).all()
    # the outgoing rows land in the old buffer, then in the rows the incoming chunks
    # freed; the last incoming chunk's rows are the next buffer and hold none of them
    last = (count - 1) // chunk * chunk
    assert nxt == in_first + last
    assert set(out_rows.tolist()) <= used and len(set(out_rows.tolist())) == count
    assert not set(out_rows.tolist()) & set(range(nxt, in_first + count))
    # swap back: the GPU slots receive the outgoing rows again, from where they landed
    if (np.diff(out_rows) == 1).all():                    # one contiguous CPU range
        g3, _, _, _ = O.chunked_swap(g2, p2, slots, int(out_rows[0]), nxt, chunk)
        assert (g3 == gpu).all()


def test_renumbered_rotary_distance_bounded():
    gd = read_golden("pace_numbers.txt")
    keep = np.sort(np.random.default_rng(16).choice(100_000, gd["budget"], replace=False))
    newp = O.renumbered_positions(len(keep), 0, keep)
    # a query continuing right after the row sees every kept token within the limit
    assert (len(keep) - newp).max() <= gd["limit"]
    assert (np.diff(newp) == 1).all()


# ---------------------------------------------------------------------------------------
# Limit rule and renumber trigger (PACE Sec. 3.2)
# ---------------------------------------------------------------------------------------

def test_limit_rule():
    gd = read_golden("pace_numbers.txt")
    for interval in (1, 512, 2048):
        assert O.smallest_limit(gd["budget"], interval, gd["prefill_chunk"]) == gd["limit"]
    assert O.smallest_limit(gd["budget"], 2049, gd["prefill_chunk"]) == 16384


def test_renumber_counts_match_pages():
    """With headroom 2,048 (reading) the per-token trigger gives the pages' counts."""
    gd = read_golden("pace_numbers.txt")
    for tokens, key in [(100_000, "renumbers_100k"), (1_000_000, "renumbers_1m"),
                        (2_000_000, "renumbers_2m")]:
        got = O.simulate_renumbers(tokens, gd["budget"], gd["limit"], 2048)
        assert abs(got / gd[key] - 1) < 0.035, (tokens, got)


def test_kv_footprint_arithmetic():
    gd = read_golden("pace_numbers.txt")
    w = synth.workload("qwen3-8b-n100k")
    assert w.kv_bytes_per_token == gd["kv_bytes_per_token"] == 144 * 1024
    assert abs(w.kv_bytes_per_token * 100_000 / 1e9 - gd["kv_gb_100k"]) < 0.05
    assert abs(w.kv_bytes_per_token * 1_000_000 / 1e9 - gd["kv_gb_1m"]) < 0.6


# ---------------------------------------------------------------------------------------
# PACE inactive equivalence (Sec. 5.7): no renumbering, no bonus == plain H2O
# ---------------------------------------------------------------------------------------

def test_inactive_equivalence_is_plain_h2o():
    w = synth.workload("qwen3-8b-n100k", n_layers=2, n_tokens=200, n_q_heads=4, n_kv_heads=2, window=8,
                       n_spans=0, budget_tokens=40)
    k, v, _ = synth.kv_cache(w, seed=2)
    q = synth.window_queries(w, seed=2)
    kl = O.gather_logical(k.float().double().numpy(), None, 16, w.n_tokens)
    vl = O.gather_logical(v.float().double().numpy(), None, 16, w.n_tokens)
    out = O.score_step(q.float().double().numpy(), kl, policy="h2o", n_sink=4, n_recent=8)
    kept, _ = O.select_items(out["item_score"], out["item_pinned"], w.budget_items)
    k2, v2, p2 = O.compact_rerope(kl, vl, kept, np.arange(w.n_tokens), -1, w.rope_theta)
    mass, _ = O.attention_mass(q.float().double().numpy(), kl)
    pin = np.zeros(w.n_tokens, bool)
    pin[:4] = pin[-8:] = True
    order = sorted([i for i in range(w.n_tokens) if not pin[i]], key=lambda i: (-mass[i], i))
    plain = sorted(list(np.nonzero(pin)[0]) + order[: w.budget_items - pin.sum()])
    assert list(kept) == plain
    assert (k2 == kl[:, plain]).all() and (v2 == vl[:, plain]).all()
    assert list(p2) == plain
