"""GPU parity of scaled RoPE tables and PACE's reference store (kv_compact_rerope_ex,
kv_compact_segment_inplace_ex, kv_ref_invalidate) against the oracle.

Bars as in test_gpu_parity: V, unrotated K, positions and store positions bit-exact;
stored keys bit-exact (they are copies); re-rotated K within 1 bf16 ulp of the oracle's
correctly rounded value.  Every step's inputs come from the oracle's own simulation.
"""
import numpy as np
import pytest
import torch

import compaction_kv_score_amd as kv
import oracle as O
from layout import unpage

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PG = 16


def ulp_bf16(x):
    """bf16 spacing at |x|, with the subnormal spacing 2**-133 at and near 0."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(x)
    return np.where(x == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def within_1ulp(got, ref):
    return bool((np.abs(np.asarray(got, np.float64) - ref) <= ulp_bf16(ref)).all())


def to_paged(logical, rng, shuffle=True, extra_pages=2):
    """[L][N][Hkv][128] values -> paged bf16 tensor [L][pages][16][Hkv][128] and block table."""
    nl, n, hkv, d = logical.shape
    n_pages = -(-n // PG)
    total = n_pages + extra_pages
    phys = rng.permutation(total)[:n_pages] if shuffle else np.arange(n_pages)
    buf = np.zeros((nl, total, PG, hkv, d))
    for p in range(n_pages):
        seg = logical[:, p * PG:(p + 1) * PG]
        buf[:, phys[p], : seg.shape[1]] = seg
    t = torch.from_numpy(buf).to(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(phys.astype(np.int32)).to(DEV) if shuffle else None
    return t, bt


def from_paged(t, bt, n):
    return unpage(t.float().cpu().double().numpy(), None if bt is None else bt.cpu().numpy(), PG, n)


def store_to_dev(ref_k, ref_pos):
    k = torch.from_numpy(np.where((ref_pos != O.REF_NONE)[None, :, None, None], ref_k, 0.0))
    return kv.RefStore(k.to(torch.bfloat16).to(DEV).contiguous(),
                       torch.from_numpy(ref_pos.astype(np.int32)).to(DEV))


@pytest.mark.parametrize("kind,kw", [
    ("linear", dict(factor=4.0)),
    ("llama3", dict(factor=8.0, original_max_position=8192, low_freq_factor=1.0, high_freq_factor=4.0)),
    ("yarn", dict(factor=16.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0)),
    ("yarn", dict(factor=4.0, original_max_position=32768, beta_fast=32.0, beta_slow=1.0, truncate=False)),
    ("yarn_ratio", dict(factor=16.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0)),
])
def test_compact_scaled_rope_parity(kind, kw):
    rng = np.random.default_rng(40)
    nl, n, hkv, n_keep = 3, 800, 2, 200
    k = O.bf16_round(rng.standard_normal((nl, n, hkv, 128)))
    v = O.bf16_round(rng.standard_normal((nl, n, hkv, 128)))
    keep = np.sort(rng.choice(n, n_keep, replace=False))
    old = (np.arange(n) + rng.integers(0, 500_000, n)).astype(np.int64)
    inv = O.scaled_inv_freq(kind, 5e5, **kw)
    rk, rv, rpos = O.compact_rerope(k, v, keep, old, 0, None, inv_freq=inv)
    kt, bt = to_paged(k, rng)
    vbuf = torch.zeros_like(kt)                      # V shares K's block table
    vl = torch.from_numpy(v).to(torch.bfloat16).to(DEV)
    for p in range(-(-n // PG)):
        phys = int(bt[p]) if bt is not None else p
        seg = vl[:, p * PG:(p + 1) * PG]
        vbuf[:, phys, : seg.shape[1]] = seg
    dk = torch.zeros((nl, -(-n_keep // PG), PG, hkv, 128), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    newp = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
    kv.kv_compact_rerope(kv.PagedCache(kt, vbuf, n, bt), kv.PagedCache(dk, dv, n_keep),
                         torch.from_numpy(keep.astype(np.int32)).to(DEV), None, n_keep,
                         torch.from_numpy(old.astype(np.int32)).to(DEV), newp, renumber_base=0,
                         rope=kv.kv_rope(kind, base=5e5, **kw))
    torch.cuda.synchronize()
    assert (newp.cpu().numpy() == rpos).all()
    assert (from_paged(dv, None, n_keep) == rv).all()
    assert within_1ulp(from_paged(dk, None, n_keep), rk)


def _state(rng, nl, n, hkv):
    """A row whose keys were cached at random positions, with an empty store."""
    k = O.bf16_round(rng.standard_normal((nl, n, hkv, 128)))
    v = O.bf16_round(rng.standard_normal((nl, n, hkv, 128)))
    pos = (np.arange(n) + rng.integers(0, 3000, n)).astype(np.int64)
    return k, v, pos, np.zeros_like(k), np.full(n, O.REF_NONE, dtype=np.int64)


def test_reference_store_sequence_parity():
    """Six compaction steps with renumbering, new tokens between steps and one planted
    stale entry; each GPU step starts from the oracle's state."""
    rng = np.random.default_rng(41)
    nl, hkv = 2, 2
    inv = O.scaled_inv_freq("default", 1e6)
    rope = kv.kv_rope("default", base=1e6)
    k, v, pos, ref_k, ref_pos = _state(rng, nl, 600, hkv)
    used_total = 0
    for step in range(6):
        n = k.shape[1]
        if step == 3:       # a slot reused without invalidation: foreign key, plausible position
            j = int(np.nonzero(ref_pos != O.REF_NONE)[0][0])
            ref_k[:, j] = O.bf16_round(rng.standard_normal((nl, hkv, 128)))
        n_keep = int(n * 0.7)
        keep = np.sort(rng.choice(n, n_keep, replace=False))
        base = int(rng.integers(0, 64))
        ok, ov, opos, oref, orefp, used = O.compact_rerope_store(k, v, keep, pos, base, inv, ref_k, ref_pos)
        used_total += int(used.sum())
        # GPU step from the same state
        kt, bt = to_paged(k, rng)
        vt = torch.zeros_like(kt)
        vl = torch.from_numpy(v).to(torch.bfloat16).to(DEV)
        for p in range(-(-n // PG)):
            phys = int(bt[p])
            seg = vl[:, p * PG:(p + 1) * PG]
            vt[:, phys, : seg.shape[1]] = seg
        src_store = store_to_dev(ref_k, ref_pos)
        dst_store = kv.RefStore.empty(nl, n_keep + 5, hkv, DEV)
        dst_store.pos.fill_(123)                      # ranks < n_keep must all be written
        dk = torch.zeros((nl, -(-n_keep // PG), PG, hkv, 128), dtype=torch.bfloat16, device=DEV)
        dv = torch.zeros_like(dk)
        newp = torch.zeros(n_keep, dtype=torch.int32, device=DEV)
        kv.kv_compact_rerope(kv.PagedCache(kt, vt, n, bt), kv.PagedCache(dk, dv, n_keep),
                             torch.from_numpy(keep.astype(np.int32)).to(DEV), None, n_keep,
                             torch.from_numpy(pos.astype(np.int32)).to(DEV), newp, renumber_base=base,
                             rope=rope, ref_src=src_store, ref_dst=dst_store)
        torch.cuda.synchronize()
        gk, gv = from_paged(dk, None, n_keep), from_paged(dv, None, n_keep)
        gp = dst_store.pos.cpu().numpy().astype(np.int64)
        assert (newp.cpu().numpy() == opos).all(), step
        assert (gv == ov).all(), step
        assert (gp[:n_keep] == orefp).all(), step
        assert (gp[n_keep:] == 123).all(), step
        valid = orefp != O.REF_NONE
        gref = dst_store.k.float().cpu().double().numpy()
        assert (gref[:, :n_keep][:, valid] == oref[:, valid]).all(), step
        assert within_1ulp(gk, ok), step
        # next state: the oracle's output plus new tokens with empty store entries
        add = 150
        k_new, v_new, _, _, _ = _state(rng, nl, add, hkv)
        k = np.concatenate([ok, k_new], axis=1)
        v = np.concatenate([ov, v_new], axis=1)
        pos = np.concatenate([opos, opos.max() + 1 + np.arange(add)])
        ref_k = np.concatenate([oref, np.zeros_like(k_new)], axis=1)
        ref_pos = np.concatenate([orefp, np.full(add, O.REF_NONE, dtype=np.int64)])
    assert used_total > 500        # later steps are served from the store


def test_segment_inplace_with_store_parity():
    rng = np.random.default_rng(42)
    nl, n, hkv, prefix, evict = 2, 1000, 2, 100, 300
    inv = O.scaled_inv_freq("llama3", 5e5, factor=8.0)
    rope = kv.kv_rope("llama3", base=5e5, factor=8.0)
    k, v, pos, ref_k, ref_pos = _state(rng, nl, n, hkv)
    # 40% of the tokens hold valid entries: the cached key is the stored key re-rotated
    has = rng.random(n) < 0.4
    for j in np.nonzero(has)[0]:
        ref_k[:, j] = O.bf16_round(rng.standard_normal((nl, hkv, 128)))
        ref_pos[j] = pos[j] - int(rng.integers(1, 5000))
        k[:, j] = O.bf16_round(O.rope_rotate(ref_k[:, j], pos[j] - ref_pos[j], inv_freq=inv))
    stale = np.nonzero(has)[0][:5]
    ref_k[:, stale] = O.bf16_round(rng.standard_normal((nl, len(stale), hkv, 128)))
    n_keep, e = kv.kv_select_segment(n, prefix, evict, PG)
    keep = O.select_segment(n, prefix, evict, PG)
    ok, ov, opos, oref, orefp, used = O.compact_rerope_store(k, v, keep, pos, 0, inv, ref_k, ref_pos)
    assert used.any() and not used[np.searchsorted(keep, stale[stale < prefix])].any()
    kt, bt = to_paged(k, rng, shuffle=False)
    vt, _ = to_paged(v, rng, shuffle=False)
    store = store_to_dev(ref_k, ref_pos)
    pos_dev = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    kv.kv_compact_segment_inplace(kv.PagedCache(kt, vt, n, bt), prefix, e, pos_dev, renumber_base=0,
                                  rope=rope, ref=store)
    torch.cuda.synchronize()
    assert (pos_dev[:n_keep].cpu().numpy() == opos).all()
    assert (from_paged(vt, bt, n)[:, :n_keep] == ov).all()
    assert within_1ulp(from_paged(kt, bt, n)[:, :n_keep], ok)
    gp = store.pos.cpu().numpy().astype(np.int64)[:n_keep]
    # a token that keeps its slot and its position keeps its entry untouched
    same = (keep == np.arange(n_keep)) & (opos == pos[keep])
    want = np.where(same, ref_pos[keep], orefp)
    assert (gp == want).all()
    valid = (want != O.REF_NONE) & ~same
    gref = store.k.float().cpu().double().numpy()[:, :n_keep]
    assert (gref[:, valid] == oref[:, valid]).all()


def test_ref_invalidate():
    st = kv.RefStore.empty(1, 300, 2, DEV)
    st.pos.copy_(torch.arange(300, dtype=torch.int32, device=DEV))
    kv.kv_ref_invalidate(st, 17, 200)
    torch.cuda.synchronize()
    p = st.pos.cpu().numpy()
    assert (p[:17] == np.arange(17)).all() and (p[17:217] == kv.KV_REF_NONE).all()
    assert (p[217:] == np.arange(217, 300)).all()
