"""C-ABI checks that need no GPU: the library loads, exports what the header declares,
and its host-only logic and argument validation follow the header's contract.

Only validation paths that return before any device call are exercised here (dummy,
never dereferenced pointers); compute parity lives in the gpu-marked tests.
"""
import ctypes

import numpy as np
import pytest

import compaction_kv_score_amd as kv
import oracle as O

FAKE = 0x10000  # 16-byte aligned dummy device address, never dereferenced here


def _cache(**over):
    d = dict(k=FAKE, v=FAKE * 2, n_layers=2, n_kv_heads=2, head_dim=128, page_size=16,
             n_tokens=100, layer_stride=7 * 16 * 2 * 128, page_stride=16 * 2 * 128,
             block_table=None)
    d.update(over)
    return kv.KvCacheDesc(**d)


def test_library_exports_every_declared_function():
    names = kv.declared_functions()
    assert len(names) >= 10
    lib = kv.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert kv.kv_abi_version() == kv.KV_ABI_VERSION == 4


def test_strerror_texts():
    for code in (kv.KV_OK, kv.KV_EINVAL, kv.KV_EUNSUPPORTED, kv.KV_EWORKSPACE, kv.KV_EHIP, kv.KV_ELIMIT):
        assert len(kv.kv_strerror(code)) >= 2
    assert "unknown" in kv.kv_strerror(12345)


@pytest.mark.parametrize("next_pos", [0, 4095, 6143, 6144, 6145, 8191, 100000])
def test_renumber_trigger_matches_oracle(next_pos):
    assert kv.kv_renumber_needed(next_pos, 2048, 8192) == O.renumber_needed(next_pos, 2048, 8192)


@pytest.mark.parametrize("n,p,e,blk", [(131072, 16384, 39322, 16), (100, 10, 7, 4), (40, 30, 50, 16),
                                       (64, 0, 0, 16), (64, 64, 5, 16), (1000, 3, 999, 64)])
def test_select_segment_host_result_matches_oracle(n, p, e, blk):
    n_keep, evict = kv.kv_select_segment(n, p, e, blk)
    assert evict == O.segment_evict_len(n, p, e, blk)
    assert n_keep == len(O.select_segment(n, p, e, blk))


def test_select_segment_rejects_bad_arguments():
    L = kv.lib()
    nk, el = ctypes.c_int64(), ctypes.c_int64()
    assert L.kv_select_segment(10, 11, 1, 16, None, 0, None, ctypes.byref(nk), ctypes.byref(el), None) == kv.KV_EINVAL
    assert L.kv_select_segment(10, 2, 1, 0, None, 0, None, ctypes.byref(nk), ctypes.byref(el), None) == kv.KV_EINVAL
    assert L.kv_select_segment(0, 0, 1, 16, None, 0, None, ctypes.byref(nk), ctypes.byref(el), None) == kv.KV_EINVAL


def _score_params(**over):
    d = dict(q=FAKE, n_q_heads=4, window=8, scale=0.0, policy=kv.KV_POLICY_H2O, item_tokens=1,
             dt_steps=1, accum=FAKE, item_score=FAKE, item_pinned=FAKE)
    d.update(over)
    return kv.KvScoreParams(**d)


def test_score_workspace_size_and_validation():
    L = kv.lib()
    n = ctypes.c_size_t()
    c, p = _cache(), _score_params()
    assert L.kv_score_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n)) == kv.KV_OK
    rows, n_lg = 2 * 8, 2 * 2
    assert n.value >= n_lg * 100 * 4 + n_lg * rows * 4  # mass partials + LSE at least
    bad = [
        (_cache(head_dim=64), p, kv.KV_EUNSUPPORTED),
        (_cache(page_size=12), p, kv.KV_EUNSUPPORTED),
        (_cache(k=None), p, kv.KV_EINVAL),
        (_cache(page_stride=100), p, kv.KV_EINVAL),
        (_cache(page_stride=1 << 32, layer_stride=1 << 33), p, kv.KV_EUNSUPPORTED),
        (c, _score_params(n_q_heads=3), kv.KV_EINVAL),
        (c, _score_params(window=101), kv.KV_EINVAL),
        (c, _score_params(window=0), kv.KV_EINVAL),
    ]
    for cc, pp, want in bad:
        assert L.kv_score_workspace_size(ctypes.byref(cc), ctypes.byref(pp), ctypes.byref(n)) == want
    # 40 query heads per KV head x 16 window rows = 640 rows > 512
    pp = _score_params(n_q_heads=80, window=16)
    assert L.kv_score_workspace_size(ctypes.byref(c), ctypes.byref(pp), ctypes.byref(n)) == kv.KV_EUNSUPPORTED


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("n_layers,hkv,hq,window,n_tokens,want_chunks", [
    (36, 8, 32, 64, 100_000, 16),      # 16 chunks of 6,272 keys: 4,608 workgroups, 9 full rounds of 512
    (36, 8, 32, 64, 1_000_000, 125),   # 125 chunks of 8,000 keys: 36,000 workgroups
    # less work (under 2,048 workgroups at 4,096 keys): the cheapest of rounds x (tiles +
    # 4), a grid of at most one workgroup per CU at 0.6 of that
    (2, 8, 32, 64, 100_000, 32),       # one full round: 32 chunks of 3,136 keys, 512 workgroups
    (8, 8, 32, 64, 30_000, 8),         # one full round: 8 chunks of 3,776 keys
    (2, 8, 32, 64, 8_000, 16),         # one workgroup per CU: 16 chunks of 512 keys
    (2, 2, 4, 8, 100, 2),              # tiny: two 64-key chunks
    (1, 2, 12, 32, 512, 8),            # Qwen2.5-1.5B head shape, one layer: 8 single-tile chunks
    (28, 2, 12, 64, 2048, 2),          # 28 layers, 384 rows in two groups: 2 chunks of 1,024 keys
])
def test_score_grid_choice(n_layers, hkv, hq, window, n_tokens, want_chunks):
    """The key chunking behind the scoring grid, read back from the workspace layout
    (LSE partials [L*Hkv][chunks][rows] float2, final LSE [L*Hkv][rows], mass partials
    [L*Hkv*row groups][N], each 256-byte aligned)."""
    L = kv.lib()
    n = ctypes.c_size_t()
    pages = -(-n_tokens // 16)
    c = _cache(n_layers=n_layers, n_kv_heads=hkv, n_tokens=n_tokens, page_stride=16 * hkv * 128,
               layer_stride=pages * 16 * hkv * 128)
    p = _score_params(n_q_heads=hq, window=window)
    assert L.kv_score_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n)) == kv.KV_OK
    units, rows = n_layers * hkv, (hq // hkv) * window
    n_rsplit = -(-rows // 256)             # row groups of at most 256, each with its own mass partial
    rest = _a256(units * rows * 4) + _a256(units * n_rsplit * n_tokens * 4)
    assert n.value == _a256(units * want_chunks * rows * 8) + rest


def test_score_group_maximum_validation():
    """The group maximum pads each group to a power of two: G = 3 with W = 150 fits as
    a sum (450 rows) but not as a maximum (4 * 150 = 600 rows); groups above 32 heads
    and unknown aggregation codes are rejected."""
    L = kv.lib()
    n = ctypes.c_size_t()
    c = _cache(n_tokens=1000, layer_stride=70 * 16 * 2 * 128)
    size = {}
    for agg in (kv.KV_AGG_SUM, kv.KV_AGG_MAX_GROUP):
        p = _score_params(n_q_heads=6, window=100, aggregate=agg)
        assert L.kv_score_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n)) == kv.KV_OK
        size[agg] = n.value
    assert size[kv.KV_AGG_MAX_GROUP] > size[kv.KV_AGG_SUM]  # 400 padded rows vs 300
    cases = [(_score_params(n_q_heads=6, window=150), kv.KV_OK),
             (_score_params(n_q_heads=6, window=150, aggregate=kv.KV_AGG_MAX_GROUP), kv.KV_EUNSUPPORTED),
             (_score_params(n_q_heads=64, window=8, aggregate=kv.KV_AGG_MAX_GROUP), kv.KV_OK),
             (_score_params(n_q_heads=66, window=4, aggregate=kv.KV_AGG_MAX_GROUP), kv.KV_EUNSUPPORTED),
             (_score_params(n_q_heads=4, window=8, aggregate=7), kv.KV_EINVAL)]
    for p, want in cases:
        assert L.kv_score_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n)) == want


def test_score_rejects_missing_state_and_small_workspace():
    L = kv.lib()
    c = _cache()
    p = _score_params(policy=kv.KV_POLICY_MEMDECAY)  # no ewma / clock / region
    assert L.kv_score(ctypes.byref(c), ctypes.byref(p), FAKE, 1 << 30, None) == kv.KV_EINVAL
    p = _score_params()
    assert L.kv_score(ctypes.byref(c), ctypes.byref(p), FAKE, 16, None) == kv.KV_EWORKSPACE
    p = _score_params(item_tokens=8)
    assert L.kv_score(ctypes.byref(c), ctypes.byref(p), FAKE, 1 << 30, None) == kv.KV_EINVAL
    # span ids need the per-span bonus table and its length
    for over in (dict(span_id=FAKE), dict(span_id=FAKE, span_bonus=FAKE),
                 dict(span_id=FAKE, n_spans=4)):
        p = _score_params(**over)
        assert L.kv_score(ctypes.byref(c), ctypes.byref(p), FAKE, 1 << 30, None) == kv.KV_EINVAL


def test_select_validation():
    L = kv.lib()
    n = ctypes.c_size_t()
    assert L.kv_select_workspace_size(1000, ctypes.byref(n)) == kv.KV_OK and n.value > 0
    assert L.kv_select_workspace_size(0, ctypes.byref(n)) == kv.KV_EINVAL
    # n_items inconsistent with n_tokens / item_tokens
    assert L.kv_select(FAKE, None, 10, 16, 100, 3, FAKE, 100, FAKE, None, FAKE, 1 << 20, None) == kv.KV_EINVAL
    assert L.kv_select(FAKE, None, 7, 16, 100, 3, FAKE, 100, FAKE, None, FAKE, 8, None) == kv.KV_EWORKSPACE
    assert L.kv_select(None, None, 7, 16, 100, 3, FAKE, 100, FAKE, None, FAKE, 1 << 20, None) == kv.KV_EINVAL


def test_compact_limit_rule_and_validation():
    """PACE Sec. 3.2: a renumbered row base + n must fit under the limit L."""
    L = kv.lib()
    src = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256)
    dst = _cache(k=FAKE * 8, v=FAKE * 16, n_tokens=4096, layer_stride=300 * 16 * 256,
                 page_stride=16 * 256)
    meta = (kv.KvMetaDesc * 1)()
    args = lambda base, maxk, limit: (ctypes.byref(src), ctypes.byref(dst), FAKE, None, maxk, FAKE,
                                      None, base, 1e6, limit, meta, 0, None)
    assert L.kv_compact_rerope(*args(0, 4096, 4095)) == kv.KV_ELIMIT
    assert L.kv_compact_rerope(*args(100, 4000, 4096)) == kv.KV_ELIMIT
    assert L.kv_compact_rerope(*args(0, 4097, 8192)) == kv.KV_EINVAL       # dst too small
    same = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256)
    assert L.kv_compact_rerope(ctypes.byref(src), ctypes.byref(same), FAKE, None, 10, FAKE, None,
                               -1, 1e6, 0, meta, 0, None) == kv.KV_EINVAL  # src == dst
    assert L.kv_compact_rerope(*args(0, 10, 0)[:8], 0.5, 0, meta, 0, None) == kv.KV_EINVAL  # theta
    bad_meta = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(FAKE, FAKE, 3, 0))
    assert L.kv_compact_rerope(*args(0, 10, 0)[:10], bad_meta, 1, None) == kv.KV_EINVAL
    assert L.kv_compact_segment_inplace(ctypes.byref(src), 100, 20, FAKE, 0, 1e4, 9000, meta, 0,
                                        None) == kv.KV_ELIMIT
    assert L.kv_compact_segment_inplace(ctypes.byref(src), 9990, 20, FAKE, 0, 1e4, 0, meta, 0,
                                        None) == kv.KV_EINVAL


def test_segment_remap_validation():
    """kv_compact_segment_remap needs a block table, whole pages and outputs of their own
    (every case is refused before anything touches the device)."""
    L = kv.lib()
    rope = kv.kv_rope("default", base=1e4)
    meta = (kv.KvMetaDesc * 1)()
    paged = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256, block_table=FAKE * 64)
    flat = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256)
    out, old, new = FAKE * 128, FAKE * 256, FAKE * 512

    def call(c, p, e, bt_out=out, freed=None, old_pos=old, new_pos=new, base=0, limit=0, m=meta, n_meta=0):
        return L.kv_compact_segment_remap(ctypes.byref(c), p, e, bt_out, freed, old_pos, new_pos, base,
                                          ctypes.byref(rope), limit, m, n_meta, None)

    assert call(flat, 160, 320) == kv.KV_EINVAL                   # no block table
    assert call(paged, 8, 320) == kv.KV_EINVAL                    # prefix not whole pages
    assert call(paged, 160, 300) == kv.KV_EINVAL                  # evicted segment not whole pages
    assert call(paged, 9984, 32) == kv.KV_EINVAL                  # past the row
    assert call(paged, 160, 320, bt_out=None) == kv.KV_EINVAL
    assert call(paged, 160, 320, bt_out=FAKE * 64 + 64) == kv.KV_EINVAL     # new table inside the old
    assert call(paged, 160, 320, freed=FAKE * 64) == kv.KV_EINVAL           # freed list over the old
    assert call(paged, 160, 320, new_pos=old + 400) == kv.KV_EINVAL         # new positions over the old
    assert call(paged, 160, 320, limit=9000) == kv.KV_ELIMIT                # 9,680 kept from 0
    bad = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(FAKE * 1024, FAKE * 1024 + 8, 4, 0))
    assert call(paged, 160, 320, m=bad, n_meta=1) == kv.KV_EINVAL          # metadata in place


def test_pages_remap_validation():
    """kv_compact_pages_remap needs a block table and outputs of its own (every case is
    refused before anything touches the device)."""
    L = kv.lib()
    rope = kv.kv_rope("default", base=1e4)
    meta = (kv.KvMetaDesc * 1)()
    paged = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256, block_table=FAKE * 64)
    flat = _cache(n_tokens=10000, layer_stride=700 * 16 * 256, page_stride=16 * 256)
    keep, out, old, new = FAKE * 2048, FAKE * 128, FAKE * 256, FAKE * 512

    def call(c, max_keep=2048, keep_=keep, bt_out=out, old_pos=old, new_pos=new, base=0, limit=0):
        return L.kv_compact_pages_remap(ctypes.byref(c), keep_, None, max_keep, bt_out, old_pos, new_pos, base,
                                        ctypes.byref(rope), limit, meta, 0, None, None)

    assert call(flat) == kv.KV_EINVAL                                  # no block table
    assert call(paged, keep_=None) == kv.KV_EINVAL
    assert call(paged, max_keep=10001) == kv.KV_EINVAL                 # more kept than the row holds
    assert call(paged, bt_out=FAKE * 64 + 16) == kv.KV_EINVAL          # new table inside the old one
    assert call(paged, new_pos=old + 40) == kv.KV_EINVAL               # new positions over the old
    assert call(paged, limit=2000) == kv.KV_ELIMIT                     # 2,048 kept from 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        kv._ptr(torch.zeros(4))


@pytest.mark.parametrize("kind,kw", [
    ("default", {}), ("linear", dict(factor=4.0)),
    ("llama3", dict(factor=8.0, original_max_position=8192, low_freq_factor=1.0, high_freq_factor=4.0)),
    ("yarn", dict(factor=16.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0)),
    ("yarn", dict(factor=4.0, original_max_position=32768, beta_fast=16.0, beta_slow=2.0, truncate=False)),
    ("yarn_ratio", dict(factor=16.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0))])
@pytest.mark.parametrize("base", [1e4, 5e5, 1e6])
def test_rope_tables_match_oracle(kind, kw, base):
    """kv_rope_inv_freq (host-only) against the oracle's scaled tables."""
    got = np.array(kv.kv_rope_inv_freq(kv.kv_rope(kind, base=base, **kw)))
    np.testing.assert_allclose(got, O.scaled_inv_freq(kind, base, **kw), rtol=1e-14, atol=0)


def test_rope_table_validation_and_explicit_table():
    L = kv.lib()
    out = (ctypes.c_double * 64)()
    for bad in (kv.kv_rope("default", base=1.0), kv.kv_rope("linear", factor=0.0),
                kv.kv_rope("llama3", factor=8.0, low_freq_factor=4.0, high_freq_factor=1.0),
                kv.kv_rope("yarn", factor=2.0, beta_fast=1.0, beta_slow=32.0),
                kv.kv_rope("yarn_ratio", factor=2.0, beta_fast=32.0, beta_slow=0.0),
                kv.kv_rope("yarn", factor=2.0, original_max_position=0),
                kv.kv_rope(7), kv.kv_rope(6), kv.kv_rope("table"),
                kv.kv_rope("table", table=[1.0] * 63 + [float("nan")])):
        assert L.kv_rope_inv_freq(ctypes.byref(bad), out) == kv.KV_EINVAL
    flags = kv.kv_rope("yarn", factor=2.0)
    flags.flags = 2                                           # no such flag
    assert L.kv_rope_inv_freq(ctypes.byref(flags), out) == kv.KV_EINVAL
    tab = [0.5 ** i for i in range(64)]
    assert kv.kv_rope_inv_freq(kv.kv_rope("table", table=tab)) == tab


def test_compact_ex_store_validation():
    L = kv.lib()
    src, dst = _cache(), _cache(k=FAKE * 3, v=FAKE * 4)
    rope = kv.kv_rope("default")
    store = lambda k, pos, n=100: kv.KvRefStore(k, pos, n, n * 2 * 128)  # noqa: E731
    a, b = store(FAKE * 5, FAKE * 6), store(FAKE * 7, FAKE * 8)
    call = lambda rs, rd, mk=10: L.kv_compact_rerope_ex(  # noqa: E731
        ctypes.byref(src), ctypes.byref(dst), FAKE, None, mk, FAKE, None, 0, ctypes.byref(rope), 0,
        None, 0, rs, rd, None)
    assert call(ctypes.byref(a), None) == kv.KV_EINVAL                        # one store only
    assert call(ctypes.byref(a), ctypes.byref(a)) == kv.KV_EINVAL             # same store twice
    small = store(FAKE * 5, FAKE * 6, n=50)
    assert call(ctypes.byref(small), ctypes.byref(b)) == kv.KV_EINVAL         # fewer slots than N
    assert call(ctypes.byref(a), ctypes.byref(store(FAKE * 7, FAKE * 8, n=5))) == kv.KV_EINVAL
    r = kv.KvRefStore(FAKE, FAKE, 100, 100 * 2 * 128)
    assert L.kv_ref_invalidate(ctypes.byref(r), 90, 20, None) == kv.KV_EINVAL
    assert L.kv_ref_invalidate(ctypes.byref(r), 0, 0, None) == kv.KV_OK


def test_lrfu_and_tail_validation():
    L = kv.lib()
    n = ctypes.c_size_t()
    assert L.kv_lrfu_workspace_size(1000, ctypes.byref(n)) == kv.KV_OK and n.value > 256
    assert L.kv_lrfu_workspace_size(0, ctypes.byref(n)) == kv.KV_EINVAL
    ok = dict(scale=1.0, top_p=0.9, decay=0.5)
    call = lambda ws, wb, **kw: L.kv_lrfu_update(FAKE, 1000, kw.get("scale", 1.0), kw.get("top_p", 0.9),  # noqa: E731
                                                kw.get("decay", 0.5), FAKE, None, ws, wb, None)
    assert call(FAKE, 16, **ok) == kv.KV_EWORKSPACE
    assert call(FAKE, 1 << 30, top_p=1.5) == kv.KV_EINVAL
    assert call(FAKE, 1 << 30, decay=-0.1) == kv.KV_EINVAL
    assert call(FAKE, 1 << 30, scale=float("inf")) == kv.KV_EINVAL
    c = _cache()
    start = ctypes.c_int64()
    assert L.kv_compact_tail_inplace(ctypes.byref(c), FAKE, None, 10, 0, None, 0, ctypes.byref(start), None,
                                     None) == kv.KV_EINVAL
    assert L.kv_compact_tail_inplace(ctypes.byref(c), None, None, 10, 50, None, 0, ctypes.byref(start), None,
                                     None) == kv.KV_EINVAL
    meta = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(FAKE, FAKE * 2, 4, 0))
    assert L.kv_compact_tail_inplace(ctypes.byref(c), FAKE, None, 10, 50, meta, 1, ctypes.byref(start), None,
                                     None) == kv.KV_EINVAL


def test_load_and_swap_validation():
    L = kv.lib()
    c = _cache()
    ws_need = ctypes.c_size_t()
    assert L.kv_offload_workspace_size(ctypes.byref(c), 64, ctypes.byref(ws_need)) == kv.KV_OK
    big = ws_need.value
    load = lambda **kw: L.kv_load_rows(  # noqa: E731
        ctypes.byref(c), kw.get("slots", FAKE), kw.get("count", 10), FAKE * 3, FAKE * 4, kw.get("rows", 50),
        kw.get("first", 0), kw.get("chunk", 64), None, 0, FAKE * 5, kw.get("wb", big), None)
    assert load(first=45) == kv.KV_EINVAL              # rows past the pool
    assert load(slots=None) == kv.KV_EINVAL
    assert load(count=-1) == kv.KV_EINVAL
    assert load(chunk=0) == kv.KV_EINVAL
    assert load(wb=big - 1) == kv.KV_EWORKSPACE
    assert load(count=0) == kv.KV_OK                   # nothing to move: no device call
    out = (ctypes.c_int64 * 10)()
    nxt = ctypes.c_int64()
    swap_ws = ctypes.c_size_t()
    assert L.kv_swap_workspace_size(ctypes.byref(c), 64, ctypes.byref(swap_ws)) == kv.KV_OK
    assert swap_ws.value == 2 * big                    # one staging area per direction
    swap = lambda **kw: L.kv_swap_chunked(  # noqa: E731
        ctypes.byref(c), FAKE, kw.get("count", 10), FAKE * 3, FAKE * 4, kw.get("rows", 100),
        kw.get("in_first", 0), kw.get("buf", 50), kw.get("chunk", 64), out, ctypes.byref(nxt), FAKE * 5,
        kw.get("wb", swap_ws.value), None, None)
    assert swap(buf=5) == kv.KV_EINVAL                 # buffer overlaps the incoming rows
    assert swap(in_first=95) == kv.KV_EINVAL
    assert swap(buf=95) == kv.KV_EINVAL                # buffer past the pool
    assert swap(wb=16) == kv.KV_EWORKSPACE
    assert swap(wb=big) == kv.KV_EWORKSPACE           # a single staging area is too small


@pytest.mark.parametrize("count,chunk,in_first,buf", [(10, 4, 0, 20), (9, 3, 30, 0), (5, 64, 7, 100),
                                                      (2048, 1024, 0, 4096), (1, 1, 3, 0)])
def test_swap_row_bookkeeping_matches_oracle(count, chunk, in_first, buf):
    """Where kv_swap_chunked reports each outgoing row lands (host logic, computed before
    any device call), against the oracle's chunk-by-chunk swap."""
    L = kv.lib()
    c = _cache(n_tokens=max(count, 100))
    rows = max(in_first + count, buf + min(chunk, count)) + 5
    ws = ctypes.c_size_t()
    assert L.kv_swap_workspace_size(ctypes.byref(c), chunk, ctypes.byref(ws)) == kv.KV_OK
    out = (ctypes.c_int64 * count)()
    nxt = ctypes.c_int64(-1)
    L.kv_swap_chunked(ctypes.byref(c), FAKE, count, FAKE * 3, FAKE * 4, rows, in_first, buf, chunk, out,
                      ctypes.byref(nxt), FAKE * 5, ws.value, None, None)
    gpu = np.zeros((1, count, 1, 1))
    pool = np.zeros((1, rows, 1, 1))
    _, _, want, want_next = O.chunked_swap(gpu, pool, np.arange(count), in_first, buf, chunk)
    assert list(out) == want.tolist() and nxt.value == want_next


def test_compact_rejects_overlapping_source_and_destination():
    """The gather form must read and write different memory: overlapping K/V extents
    (caches without a block table), positions or metadata are refused on the host."""
    L = kv.lib()
    G = 1 << 30                                           # far-apart fake bases, never dereferenced
    src = _cache(k=G, v=2 * G, n_tokens=1000)
    ok_dst = _cache(k=3 * G, v=4 * G, n_tokens=100)
    span = 2 * (7 * 16 * 2 * 128 + 63 * 16 * 2 * 128)     # bytes of src's K extent
    inside = _cache(k=G + span - 256, v=4 * G, n_tokens=100)
    after = _cache(k=G + span, v=4 * G, n_tokens=100)
    meta0 = (kv.KvMetaDesc * 1)()

    def call(dst, old=5 * G, new=6 * G, meta=meta0, n_meta=0):
        return L.kv_compact_rerope(ctypes.byref(src), ctypes.byref(dst), FAKE, None, 100, old, new, 0, 1e6, 0,
                                   meta, n_meta, None)
    # validation passes and the call reaches the device check (no GPU here)
    assert call(ok_dst) not in (kv.KV_EINVAL, kv.KV_ELIMIT, kv.KV_EWORKSPACE)
    assert call(after) not in (kv.KV_EINVAL, kv.KV_ELIMIT, kv.KV_EWORKSPACE)
    assert call(inside) == kv.KV_EINVAL                   # dst K inside src K's extent
    assert call(_cache(k=3 * G, v=2 * G + 512, n_tokens=100)) == kv.KV_EINVAL   # dst V inside src V
    assert call(ok_dst, old=5 * G, new=5 * G + 3996) == kv.KV_EINVAL          # new_pos over old_pos
    assert call(ok_dst, old=5 * G, new=5 * G + 4000) not in (kv.KV_EINVAL,)
    m = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(7 * G, 7 * G + 3000, 4, 0))         # dst inside src
    assert call(ok_dst, meta=m, n_meta=1) == kv.KV_EINVAL
    m = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(7 * G, 6 * G + 200, 4, 0))          # dst over new_pos
    assert call(ok_dst, meta=m, n_meta=1) == kv.KV_EINVAL
    m = (kv.KvMetaDesc * 1)(kv.KvMetaDesc(7 * G, 8 * G, 4, 0))
    assert call(ok_dst, meta=m, n_meta=1) not in (kv.KV_EINVAL,)
