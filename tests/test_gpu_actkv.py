"""GPU parity of ActKV's LRFU keep scores (top-p hit mask) and in-place tail compaction
(kv_lrfu_update, kv_compact_tail_inplace) against the oracle.

Bars: hit masks, moved slots, metadata and status bit-exact (the top-p set is decided
from exact sums of the float32 scores on both sides: rationals in the oracle, multi-word
integers on the device); keep scores within 1e-6 relative (float32 update against
float64).
"""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
from layout import unpage

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _scores(rng, n, dist):
    if dist == "power":
        return (rng.random(n) ** 8).astype(np.float32)
    if dist == "ties":
        return (rng.integers(0, 6, n) / 8.0).astype(np.float32)
    if dist == "mixed":
        s = (rng.random(n) ** 3).astype(np.float32)
        s[rng.random(n) < 0.1] = 0.0
        s[rng.random(n) < 0.05] = -0.0
        s[rng.random(n) < 0.05] = -1.0
        s[rng.random(n) < 0.01] = np.nan
        return s
    if dist == "equal":
        return np.full(n, 0.125, np.float32)
    if dist == "tiny":
        return (rng.random(n) * 1e-30).astype(np.float32)
    if dist == "wide":
        # 10^U(-45, 0): normal and subnormal float32 scores over the whole range
        s = np.power(10.0, rng.uniform(-45.0, 0.0, n)).astype(np.float32)
        s[rng.random(n) < 0.05] = 0.0
        return s
    if dist == "twobinade":
        # one dominant score and many others from a single small exponent: the boundary
        # falls among equal-exponent scores far below the largest
        s = (1.0 + rng.random(n)).astype(np.float32) * np.float32(2.0 ** -100)
        s[0] = 1.0
        return s
    raise ValueError(dist)


@pytest.mark.parametrize("n,dist,p,scale", [
    (1, "power", 0.9, 1.0),
    (100, "ties", 0.9, 1.0),
    (5000, "mixed", 0.9, 1.0),
    (5000, "equal", 0.5, 1.0),
    (9000, "tiny", 0.9, 1.0),
    (100_000, "power", 0.9, 1.0 / (36 * 8 * 64)),
    (100_000, "ties", 1.0, 1.0),
    (100_000, "mixed", 0.0, 1.0),
    (262_147, "power", 0.999, 3.0),
    (5000, "wide", 1.0, 1.0),                     # every positive score is a hit
    (5000, "wide", 0.999, 1.0),
    (100_000, "wide", 0.9, 1.0),
    (70_000, "wide", 1.0, 1e-20),                 # products underflow to subnormals and 0
    (4097, "twobinade", 1.0, 1.0),
    (4097, "twobinade", float(np.nextafter(np.float32(1.0), np.float32(0.0))), 1.0),
    (131_072, "mixed", 0.9, 1.0),                 # 64 full blocks of 2,048 entries
    (131_073, "wide", 0.999, 1.0),                # 64 blocks of 2,049 (the last one short)
    (1_048_583, "power", 0.9, 1.0),               # the largest block count, ragged tail
    (1_048_583, "ties", 0.75, 1.0),
    # rows of at most 4,096 entries take the one-block kernel
    (4096, "mixed", 0.9, 1.0),
    (4096, "mixed", 0.0, 1.0),
    (4096, "wide", 1.0, 1.0),
    (4096, "wide", 0.999, 1.0),
    (4096, "twobinade", 1.0, 1.0),
    (4096, "twobinade", float(np.nextafter(np.float32(1.0), np.float32(0.0))), 1.0),
    (3000, "tiny", 0.9, 1.0),
    (2000, "equal", 0.5, 1.0),
    (2500, "wide", 1.0, 1e-20),
])
def test_lrfu_update_parity(n, dist, p, scale):
    rng = np.random.default_rng(n + len(dist))
    a = _scores(rng, n, dist)
    ks0 = (rng.random(n) * 2).astype(np.float32)
    s = (a * np.float32(scale)).astype(np.float32)                # the float32 product the kernel forms
    ks_ref, hit_ref = O.lrfu_update(ks0.astype(np.float64), s, p=p, decay=0.5)
    ks = torch.from_numpy(ks0).to(DEV)
    hit = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
    kv.kv_lrfu_update(torch.from_numpy(a).to(DEV), ks, scale=scale, top_p=p, decay=0.5, hit=hit)
    torch.cuda.synchronize()
    got_hit = hit.cpu().numpy().astype(bool)
    assert (got_hit == hit_ref).all(), (int((got_hit != hit_ref).sum()), int(hit_ref.sum()))
    np.testing.assert_allclose(ks.cpu().numpy().astype(np.float64), ks_ref, rtol=1e-6, atol=1e-37)


def test_lrfu_steps_then_select():
    """Five LRFU steps with new entries appended at KS = 0, then TopK by kv_select."""
    rng = np.random.default_rng(7)
    n, budget = 3000, 400
    ks_ref = np.zeros(n)
    ks = torch.zeros(n, device=DEV)
    for step in range(5):
        a = _scores(rng, n, "power")
        ks_ref, _ = O.lrfu_update(ks_ref, a, p=0.9, decay=0.5)
        kv.kv_lrfu_update(torch.from_numpy(a).to(DEV), ks, top_p=0.9, decay=0.5)
        add = 200
        ks_ref = np.concatenate([ks_ref, np.zeros(add)])
        ks = torch.cat([ks, torch.zeros(add, device=DEV)])
        n += add
    torch.cuda.synchronize()
    np.testing.assert_allclose(ks.cpu().numpy().astype(np.float64), ks_ref, rtol=1e-5, atol=1e-30)
    keep = torch.zeros(budget, dtype=torch.int32, device=DEV)
    nk = torch.zeros(1, dtype=torch.int64, device=DEV)
    kv.kv_select(ks, None, 1, n, budget, keep, nk)
    torch.cuda.synchronize()
    # the oracle selects on its own keep scores; the sets may differ only in entries whose
    # oracle score lies within 1e-5 relative of the oracle's selection threshold
    want, _ = O.select_items(ks_ref.astype(np.float32), None, budget)
    got = keep.cpu().numpy()
    assert int(nk) == budget
    thr = np.sort(ks_ref)[::-1][budget - 1]
    diff = np.setxor1d(got, want)
    assert (np.abs(ks_ref[diff] - thr) <= 1e-5 * abs(thr)).all(), diff


def _paged(rng, logical, shuffle):
    nl, slots, hkv, d = logical.shape
    pages = slots // 16
    phys = rng.permutation(pages + 3)[:pages] if shuffle else np.arange(pages)
    buf = torch.zeros((nl, pages + 3, 16, hkv, d), dtype=torch.bfloat16)
    lt = torch.from_numpy(logical).to(torch.bfloat16)
    for p in range(pages):
        buf[:, phys[p]] = lt[:, p * 16:(p + 1) * 16]
    bt = torch.from_numpy(phys.astype(np.int32)).to(DEV) if shuffle else None
    return buf.to(DEV), bt


def _logical(t, bt, slots):
    return unpage(t.float().cpu().double().numpy(), None if bt is None else bt.cpu().numpy(), 16, slots)


@pytest.mark.parametrize("n,budget,n_keep,shuffle,dev_count,nl,hkv", [
    (1000, 300, 300, True, False, 2, 2),     # region reaches past N into the last block
    (1024, 256, 200, False, True, 2, 2),     # fewer kept than the budget, device count
    (777, 100, 100, True, False, 2, 2),
    (5000, 2048, 2048, True, True, 2, 2),
    (64, 16, 16, False, False, 2, 2),
    (500, 600, 300, True, False, 2, 2),      # budget above N: nothing moves
    (3000, 1024, 1000, True, True, 9, 4),    # 576 chunk pairs per token, many layers and heads
])
def test_tail_compact_parity(n, budget, n_keep, shuffle, dev_count, nl, hkv):
    rng = np.random.default_rng(n + budget)
    slots = -(-n // 16) * 16
    k = O.bf16_round(rng.standard_normal((nl, slots, hkv, 128)))
    v = O.bf16_round(rng.standard_normal((nl, slots, hkv, 128)))
    pos = rng.integers(0, 2 ** 31 - 1, slots).astype(np.int32)
    sc = rng.random(slots).astype(np.float32)
    keep = np.sort(rng.choice(n, min(n_keep, n), replace=False))
    kt, bt = _paged(rng, k, shuffle)
    vt = torch.zeros_like(kt)
    vt_l, _ = _paged(np.random.default_rng(0), v, False)
    # V shares K's block table
    for p in range(slots // 16):
        phys = int(bt[p]) if bt is not None else p
        vt[:, phys] = vt_l[:, p]
    pos_d, sc_d = torch.from_numpy(pos).to(DEV), torch.from_numpy(sc).to(DEV)
    keep_d = torch.from_numpy(np.concatenate([keep, [0] * 5]).astype(np.int32)).to(DEV)
    cnt = torch.tensor([len(keep)], dtype=torch.int64, device=DEV) if dev_count else None
    max_keep = len(keep) + (5 if dev_count else 0)
    status = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    start = kv.kv_compact_tail_inplace(kv.PagedCache(kt, vt, n, bt), keep_d, cnt, max_keep if dev_count else len(keep),
                                       budget, meta=[pos_d, sc_d], status=status)
    torch.cuda.synchronize()
    if budget >= n:
        assert start == 0
        src = dst = np.zeros(0, dtype=np.int64)
    else:
        s0, e0, src, dst, over = O.tail_compaction_pairs(n, keep, budget, 16)
        assert start == s0 and not over
    assert int(status.item()) == 0
    assert (_logical(kt, bt, slots) == O.tail_compact(k, src, dst)).all()
    assert (_logical(vt, bt, slots) == O.tail_compact(v, src, dst)).all()
    assert (pos_d.cpu().numpy() == O.tail_compact(pos[None], src, dst)[0]).all()
    assert (sc_d.cpu().numpy() == O.tail_compact(sc[None], src, dst)[0]).all()


def test_tail_compact_overflow_status():
    rng = np.random.default_rng(5)
    n, budget = 640, 100
    keep = np.sort(rng.choice(n, 130, replace=False))          # more kept than the budget
    k = O.bf16_round(rng.standard_normal((1, n, 1, 128)))
    kt, _ = _paged(rng, k, False)
    vt = kt.clone()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kv_compact_tail_inplace(kv.PagedCache(kt, vt, n), torch.from_numpy(keep.astype(np.int32)).to(DEV), None,
                               len(keep), budget, status=status)
    torch.cuda.synchronize()
    s0, e0, src, dst, over = O.tail_compaction_pairs(n, keep, budget, 16)
    assert over and int(status.item()) == kv.KV_STATUS_KEEP_OVERFLOW
    assert (_logical(kt, None, n) == O.tail_compact(k, src, dst)).all()
