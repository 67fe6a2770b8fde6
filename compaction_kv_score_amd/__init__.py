"""Python binding of libkvscore (MI355X / gfx950 KV-cache scoring, selection,
compaction and exact re-rotation).

This module only marshals arguments: it turns torch tensors into device pointers and
sizes, passes the current HIP stream, and raises on error codes.  Every step of the
path runs in the HIP kernels of libkvscore.so; there is no fallback.  The functions
carry the names of the C entry points declared in include/kvscore.h, whose comments
document arguments, layouts, ownership and errors.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVSCORE_LIB names another build of the same library (the tests load the host-sanitized
# build this way); by default the library built in place next to this file is loaded.
LIB_PATH = os.environ.get("KVSCORE_LIB") or os.path.join(_PKG, "libkvscore.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kvscore.h")

KV_OK = 0
KV_EINVAL = -1
KV_EUNSUPPORTED = -2
KV_EWORKSPACE = -3
KV_EHIP = -4
KV_ELIMIT = -5
KV_STATUS_PINNED_OVER_BUDGET = 1
KV_STATUS_NAN_SCORE = 2
KV_STATUS_KEEP_OVERFLOW = 4
KV_STATUS_BAD_REGION = 8
KV_STATUS_NOT_WHOLE_PAGES = 16
KV_POLICY_MEMDECAY = 0
KV_POLICY_H2O = 1
KV_AGG_SUM = 0
KV_AGG_MAX_GROUP = 1
KV_ROPE_DEFAULT = 0
KV_ROPE_LINEAR = 1
KV_ROPE_LLAMA3 = 2
KV_ROPE_YARN = 3
KV_ROPE_TABLE = 4
KV_ROPE_YARN_RATIO = 5
KV_ROPE_YARN_NO_TRUNCATE = 1
KV_REF_NONE = -(2 ** 31)
KV_MAX_META = 8
KV_ABI_VERSION = 4  # layout of the structs below


class KvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kv_strerror(code)} (code {code})")


class KvCacheDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_tokens", ctypes.c_int64), ("layer_stride", ctypes.c_int64),
                ("page_stride", ctypes.c_int64), ("block_table", ctypes.c_void_p)]


class KvMetaDesc(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p),
                ("elem_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KvScoreParams(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("n_q_heads", ctypes.c_int32),
                ("window", ctypes.c_int32), ("scale", ctypes.c_float),
                ("policy", ctypes.c_int32), ("item_tokens", ctypes.c_int32),
                ("dt_steps", ctypes.c_int32), ("lse_in", ctypes.c_void_p),
                ("region", ctypes.c_void_p), ("base_prio", ctypes.c_void_p),
                ("decay_rate", ctypes.c_void_p), ("n_regions", ctypes.c_int32),
                ("rho", ctypes.c_float), ("alpha", ctypes.c_float), ("tau", ctypes.c_float),
                ("ewma", ctypes.c_void_p), ("clock", ctypes.c_void_p),
                ("accum", ctypes.c_void_p), ("span_id", ctypes.c_void_p),
                ("span_bonus", ctypes.c_void_p), ("n_spans", ctypes.c_int32),
                ("pinned_regions", ctypes.c_uint32),
                ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("token_pinned", ctypes.c_void_p), ("mass", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("token_score", ctypes.c_void_p),
                ("item_score", ctypes.c_void_p), ("item_pinned", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p), ("aggregate", ctypes.c_int32),
                ("status", ctypes.c_void_p)]


class KvRope(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("original_max_position", ctypes.c_int32),
                ("base", ctypes.c_double), ("factor", ctypes.c_double),
                ("low_freq_factor", ctypes.c_double), ("high_freq_factor", ctypes.c_double),
                ("beta_fast", ctypes.c_double), ("beta_slow", ctypes.c_double),
                ("inv_freq", ctypes.POINTER(ctypes.c_double)), ("flags", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class KvRefStore(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("n_slots", ctypes.c_int64),
                ("layer_stride", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvscore.so (built in place by compaction_kv_score_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compaction_kv_score_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER
        sigs = {
            "kv_abi_version": (i32, []),
            "kv_strerror": (ctypes.c_char_p, [i32]),
            "kv_renumber_needed": (i32, [i64, i32, i32]),
            "kv_score_workspace_size": (i32, [P(KvCacheDesc), P(KvScoreParams), P(sz)]),
            "kv_score": (i32, [P(KvCacheDesc), P(KvScoreParams), vp, sz, vp]),
            "kv_select_workspace_size": (i32, [i64, P(sz)]),
            "kv_select": (i32, [vp, vp, i64, i32, i64, i64, vp, i64, vp, vp, vp, sz, vp]),
            "kv_select_noalloc": (i32, [vp, vp, i64, i32, i64, i64, vp, i64, vp, vp, vp]),
            "kv_select_segment": (i32, [i64, i64, i64, i32, vp, i64, vp, P(i64), P(i64), vp]),
            "kv_compact_rerope": (i32, [P(KvCacheDesc), P(KvCacheDesc), vp, vp, i64, vp, vp, i32,
                                        ctypes.c_double, i32, P(KvMetaDesc), i32, vp]),
            "kv_compact_segment_inplace": (i32, [P(KvCacheDesc), i64, i64, vp, i32, ctypes.c_double,
                                                 i32, P(KvMetaDesc), i32, vp]),
            "kv_rope_inv_freq": (i32, [P(KvRope), P(ctypes.c_double)]),
            "kv_lrfu_workspace_size": (i32, [i64, P(sz)]),
            "kv_gather_evicted": (i32, [P(KvCacheDesc), vp, i64, i64, i64, P(KvCacheDesc), vp, P(KvMetaDesc),
                                        i32, vp]),
            "kv_offload_workspace_size": (i32, [P(KvCacheDesc), i64, P(sz)]),
            "kv_offload_evicted": (i32, [P(KvCacheDesc), vp, i64, i64, vp, vp, vp, vp, sz, vp]),
            "kv_load_rows": (i32, [P(KvCacheDesc), vp, i64, vp, vp, i64, i64, i64, P(KvMetaDesc), i32, vp,
                                   sz, vp]),
            "kv_swap_workspace_size": (i32, [P(KvCacheDesc), i64, P(sz)]),
            "kv_swap_chunked": (i32, [P(KvCacheDesc), vp, i64, vp, vp, i64, i64, i64, i64, P(i64), P(i64), vp,
                                      sz, vp, vp]),
            "kv_lrfu_update": (i32, [vp, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float, vp, vp, vp, sz,
                                     vp]),
            "kv_compact_tail_inplace": (i32, [P(KvCacheDesc), vp, vp, i64, i64, P(KvMetaDesc), i32, P(i64),
                                              vp, vp]),
            "kv_ref_invalidate": (i32, [P(KvRefStore), i64, i64, vp]),
            "kv_compact_rerope_ex": (i32, [P(KvCacheDesc), P(KvCacheDesc), vp, vp, i64, vp, vp, i32,
                                           P(KvRope), i32, P(KvMetaDesc), i32, P(KvRefStore),
                                           P(KvRefStore), vp]),
            "kv_compact_segment_inplace_ex": (i32, [P(KvCacheDesc), i64, i64, vp, i32, P(KvRope), i32,
                                                    P(KvMetaDesc), i32, P(KvRefStore), vp]),
            "kv_compact_segment_remap": (i32, [P(KvCacheDesc), i64, i64, vp, vp, vp, vp, i32, P(KvRope), i32,
                                               P(KvMetaDesc), i32, vp]),
            "kv_compact_pages_remap": (i32, [P(KvCacheDesc), vp, vp, i64, vp, vp, vp, i32, P(KvRope), i32,
                                             P(KvMetaDesc), i32, vp, vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.kv_abi_version() != KV_ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.kv_abi_version()}, this binding "
                               f"expects {KV_ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/kvscore.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char \*)\s*(kv_\w+)\s*\(", text, re.M)))


# ------------------------------------------------------------------------- marshalling
def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("tensors passed to libkvscore must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkvscore must be contiguous")
    return t.data_ptr()


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(code: int, where: str):
    if code < 0:
        raise KvError(code, where)
    return code


def kv_abi_version() -> int:
    return lib().kv_abi_version()


def kv_strerror(code: int) -> str:
    return lib().kv_strerror(code).decode()


def kv_renumber_needed(next_pos: int, headroom: int, limit: int) -> bool:
    return bool(lib().kv_renumber_needed(next_pos, headroom, limit))


class PagedCache:
    """A paged KV cache row held in two torch tensors of shape
    [layers][physical pages][page_size][kv_heads][head_dim] (bf16, contiguous) plus an
    optional int32 block table; n_tokens logical tokens are in use."""

    def __init__(self, k, v, n_tokens, block_table=None):
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or k.shape != v.shape:
            raise ValueError("k and v must be bf16 tensors of the same shape")
        if k.dim() != 5:
            raise ValueError("k and v must be [layers][pages][page_size][kv_heads][head_dim]")
        self.k, self.v, self.block_table = k, v, block_table
        self.n_tokens = int(n_tokens)
        nl, npg, ps, hk, d = k.shape
        self.n_layers, self.n_phys_pages, self.page_size, self.n_kv_heads, self.head_dim = nl, npg, ps, hk, d
        if block_table is not None and block_table.dtype != torch.int32:
            raise ValueError("block_table must be int32")

    def desc(self) -> KvCacheDesc:
        nl, npg, ps, hk, d = self.k.shape
        return KvCacheDesc(_ptr(self.k), _ptr(self.v), nl, hk, d, ps, self.n_tokens,
                           npg * ps * hk * d, ps * hk * d, _ptr(self.block_table))


def _meta_array(meta):
    meta = list(meta or [])
    if len(meta) > KV_MAX_META:
        raise ValueError("too many metadata arrays")
    arr = (KvMetaDesc * max(1, len(meta)))()
    for i, (src, dst) in enumerate(meta):
        arr[i] = KvMetaDesc(_ptr(src), _ptr(dst), src.element_size(), 0)
    return arr, len(meta)


def _score_params(q, *, policy, window, item_tokens, scale=0.0, dt_steps=1, lse_in=None,
                  region=None, base_prio=None, decay_rate=None, rho=0.9, alpha=1.0, tau=0.01,
                  ewma=None, clock=None, accum=None, span_id=None, span_bonus=None,
                  pinned_regions=0, n_sink=0, n_recent=0,
                  token_pinned=None, mass=None, lse=None, token_score=None, item_score=None,
                  item_pinned=None, stage_events=None, aggregate="sum", status=None):
    pol = {"memdecay": KV_POLICY_MEMDECAY, "h2o": KV_POLICY_H2O}.get(policy, policy)
    agg = {"sum": KV_AGG_SUM, "max_group": KV_AGG_MAX_GROUP}.get(aggregate, aggregate)
    n_regions = int(base_prio.numel()) if base_prio is not None else 0
    if span_bonus is not None and span_bonus.dtype != torch.float32:
        raise TypeError("span_bonus must be float32")
    n_spans = int(span_bonus.numel()) if span_bonus is not None else 0
    return KvScoreParams(
        _ptr(q), int(q.shape[2]), int(window), float(scale), int(pol), int(item_tokens),
        int(dt_steps), _ptr(lse_in), _ptr(region), _ptr(base_prio), _ptr(decay_rate), n_regions,
        float(rho), float(alpha), float(tau), _ptr(ewma), _ptr(clock), _ptr(accum),
        _ptr(span_id), _ptr(span_bonus), n_spans, int(pinned_regions),
        int(n_sink), int(n_recent), _ptr(token_pinned), _ptr(mass), _ptr(lse),
        _ptr(token_score), _ptr(item_score), _ptr(item_pinned), stage_events, int(agg),
        _ptr(status))


def kv_score_workspace_size(cache: PagedCache, q, **kw) -> int:
    p = _score_params(q, **kw)
    n = ctypes.c_size_t(0)
    _check(lib().kv_score_workspace_size(ctypes.byref(cache.desc()), ctypes.byref(p), ctypes.byref(n)),
           "kv_score_workspace_size")
    return n.value


def kv_score(cache: PagedCache, q, workspace=None, **kw):
    """Score the cache row (see kv_score in include/kvscore.h); keyword arguments are the
    fields of kv_score_params (tensors on the device, scalars as Python numbers)."""
    p = _score_params(q, **kw)
    d = cache.desc()
    if workspace is None:
        workspace = torch.empty(kv_score_workspace_size(cache, q, **kw), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv_score(ctypes.byref(d), ctypes.byref(p), _ptr(workspace), workspace.numel(),
                          _stream(q.device)), "kv_score")
    return workspace


def kv_select_workspace_size(n_items: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kv_select_workspace_size(int(n_items), ctypes.byref(n)), "kv_select_workspace_size")
    return n.value


def kv_select(item_score, item_pinned, item_tokens, n_tokens, budget_items, keep_tokens, n_keep,
              status=None, workspace=None):
    """Budget selection (see kv_select in include/kvscore.h)."""
    n_items = int(item_score.numel())
    if workspace is None:
        workspace = torch.empty(kv_select_workspace_size(n_items), dtype=torch.uint8,
                                device=item_score.device)
    _check(lib().kv_select(_ptr(item_score), _ptr(item_pinned), n_items, int(item_tokens),
                           int(n_tokens), int(budget_items), _ptr(keep_tokens), keep_tokens.numel(),
                           _ptr(n_keep), _ptr(status), _ptr(workspace), workspace.numel(),
                           _stream(item_score.device)), "kv_select")
    return workspace


def kv_select_noalloc(item_score, item_pinned, item_tokens, n_tokens, budget_items, keep_tokens, n_keep,
                      status=None):
    """Budget selection in the library's fixed device scratch (see kv_select_noalloc)."""
    _check(lib().kv_select_noalloc(_ptr(item_score), _ptr(item_pinned), int(item_score.numel()),
                                   int(item_tokens), int(n_tokens), int(budget_items), _ptr(keep_tokens),
                                   keep_tokens.numel(), _ptr(n_keep), _ptr(status),
                                   _stream(item_score.device)), "kv_select_noalloc")


def kv_lrfu_workspace_size(n: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().kv_lrfu_workspace_size(int(n), ctypes.byref(b)), "kv_lrfu_workspace_size")
    return b.value


def kv_lrfu_update(attn_score, keep_score, scale=1.0, top_p=0.9, decay=0.5, hit=None, workspace=None):
    """ActKV LRFU keep-score step (see kv_lrfu_update in include/kvscore.h)."""
    n = int(attn_score.numel())
    if workspace is None:
        workspace = torch.empty(kv_lrfu_workspace_size(n), dtype=torch.uint8, device=attn_score.device)
    _check(lib().kv_lrfu_update(_ptr(attn_score), n, float(scale), float(top_p), float(decay),
                                _ptr(keep_score), _ptr(hit), _ptr(workspace), workspace.numel(),
                                _stream(attn_score.device)), "kv_lrfu_update")
    return workspace


def kv_gather_evicted(src: PagedCache, keep_tokens, n_keep, first, count, dst: PagedCache,
                      evicted_tokens=None, meta=None):
    """Gather evicted rows (see kv_gather_evicted); n_keep is a host count; meta is a list
    of (src, dst) tensor pairs."""
    arr, n_meta = _meta_array(meta)
    _check(lib().kv_gather_evicted(ctypes.byref(src.desc()), _ptr(keep_tokens), int(n_keep), int(first),
                                   int(count), ctypes.byref(dst.desc()), _ptr(evicted_tokens), arr, n_meta,
                                   _stream(src.k.device)), "kv_gather_evicted")


def _host_ptr(t):
    if t is None:
        return None
    if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
        raise ValueError("host buffers must be contiguous pinned CPU tensors")
    return t.data_ptr()


def kv_offload_evicted(src: PagedCache, keep_tokens, n_keep, host_k, host_v, host_tokens=None, chunk=1024,
                       workspace=None):
    """Offload every evicted row to pinned host tensors (see kv_offload_evicted)."""
    d = src.desc()
    if workspace is None:
        b = ctypes.c_size_t(0)
        _check(lib().kv_offload_workspace_size(ctypes.byref(d), int(chunk), ctypes.byref(b)),
               "kv_offload_workspace_size")
        workspace = torch.empty(b.value, dtype=torch.uint8, device=src.k.device)
    _check(lib().kv_offload_evicted(ctypes.byref(d), _ptr(keep_tokens), int(n_keep), int(chunk),
                                    _host_ptr(host_k), _host_ptr(host_v), _host_ptr(host_tokens),
                                    _ptr(workspace), workspace.numel(), _stream(src.k.device)),
           "kv_offload_evicted")
    return workspace


def kv_offload_workspace_size(cache: PagedCache, chunk) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().kv_offload_workspace_size(ctypes.byref(cache.desc()), int(chunk), ctypes.byref(b)),
           "kv_offload_workspace_size")
    return b.value


def kv_load_rows(dst: PagedCache, slots, host_k, host_v, host_first=0, count=None, chunk=1024, meta=None,
                 workspace=None):
    """Host rows [host_first, host_first + count) of pinned pools [L][rows][Hkv][128] into
    slots `slots` of dst (see kv_load_rows); meta is a list of (src[count], dst[N]) pairs."""
    count = int(slots.numel()) if count is None else int(count)
    if workspace is None:
        workspace = torch.empty(kv_offload_workspace_size(dst, chunk), dtype=torch.uint8, device=dst.k.device)
    arr, n_meta = _meta_array(meta)
    _check(lib().kv_load_rows(ctypes.byref(dst.desc()), _ptr(slots), count, _host_ptr(host_k), _host_ptr(host_v),
                              int(host_k.shape[1]), int(host_first), int(chunk), arr, n_meta, _ptr(workspace),
                              workspace.numel(), _stream(dst.k.device)), "kv_load_rows")
    return workspace


def kv_swap_workspace_size(cache: PagedCache, chunk) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().kv_swap_workspace_size(ctypes.byref(cache.desc()), int(chunk), ctypes.byref(b)),
           "kv_swap_workspace_size")
    return b.value


def kv_swap_chunked(cache: PagedCache, slots, host_k, host_v, in_first, buf_first, chunk=1024, workspace=None,
                    in_stream=None):
    """Penelope's both-tiers-full swap (see kv_swap_chunked): the outgoing side runs on the
    current stream, the incoming side on in_stream (a torch.cuda.Stream; None = the current
    stream, everything in order).  Returns (out_rows list, next_buf_first, workspace)."""
    count = int(slots.numel())
    if workspace is None:
        workspace = torch.empty(kv_swap_workspace_size(cache, chunk), dtype=torch.uint8, device=cache.k.device)
    out = (ctypes.c_int64 * max(1, count))()
    nxt = ctypes.c_int64(-1)
    s = _stream(cache.k.device)
    s_in = s if in_stream is None else ctypes.c_void_p(in_stream.cuda_stream)
    _check(lib().kv_swap_chunked(ctypes.byref(cache.desc()), _ptr(slots), count, _host_ptr(host_k),
                                 _host_ptr(host_v), int(host_k.shape[1]), int(in_first), int(buf_first),
                                 int(chunk), out, ctypes.byref(nxt), _ptr(workspace), workspace.numel(),
                                 s, s_in), "kv_swap_chunked")
    return list(out)[:count], nxt.value, workspace


def kv_compact_tail_inplace(cache: PagedCache, keep_tokens, n_keep, max_keep, budget, meta=None,
                            status=None) -> int:
    """ActKV in-place tail compaction (see kv_compact_tail_inplace); meta is a list of
    tensors moved in place.  Returns the first slot of the target region."""
    arr, n_meta = _meta_array([(m, m) for m in (meta or [])])
    start = ctypes.c_int64(0)
    _check(lib().kv_compact_tail_inplace(ctypes.byref(cache.desc()), _ptr(keep_tokens), _ptr(n_keep),
                                         int(max_keep), int(budget), arr, n_meta, ctypes.byref(start),
                                         _ptr(status), _stream(cache.k.device)), "kv_compact_tail_inplace")
    return start.value


def kv_select_segment(n_tokens, prefix_len, evict_tokens, block, keep_tokens=None, n_keep_dev=None):
    """Penelope segment (see kv_select_segment); returns (n_keep, evict_len)."""
    nk, el = ctypes.c_int64(0), ctypes.c_int64(0)
    dev = keep_tokens.device if keep_tokens is not None else (
        n_keep_dev.device if n_keep_dev is not None else None)
    stream = _stream(dev) if dev is not None else None
    _check(lib().kv_select_segment(int(n_tokens), int(prefix_len), int(evict_tokens), int(block),
                                   _ptr(keep_tokens),
                                   keep_tokens.numel() if keep_tokens is not None else 0,
                                   _ptr(n_keep_dev), ctypes.byref(nk), ctypes.byref(el), stream),
           "kv_select_segment")
    return nk.value, el.value


def kv_rope(kind="default", base=1e6, factor=1.0, original_max_position=8192, low_freq_factor=1.0,
            high_freq_factor=4.0, beta_fast=32.0, beta_slow=1.0, table=None, truncate=True) -> KvRope:
    """A kv_rope descriptor (see include/kvscore.h); kind is a name or a KV_ROPE_* code;
    truncate=False sets KV_ROPE_YARN_NO_TRUNCATE."""
    code = {"default": KV_ROPE_DEFAULT, "linear": KV_ROPE_LINEAR, "llama3": KV_ROPE_LLAMA3,
            "yarn": KV_ROPE_YARN, "yarn_ratio": KV_ROPE_YARN_RATIO, "table": KV_ROPE_TABLE}.get(kind, kind)
    r = KvRope(int(code), int(original_max_position), float(base), float(factor), float(low_freq_factor),
               float(high_freq_factor), float(beta_fast), float(beta_slow), None,
               0 if truncate else KV_ROPE_YARN_NO_TRUNCATE, 0)
    if table is not None:
        arr = (ctypes.c_double * 64)(*[float(x) for x in table])
        r._table = arr                      # keep the host array alive with the struct
        r.inv_freq = ctypes.cast(arr, ctypes.POINTER(ctypes.c_double))
    return r


def kv_rope_inv_freq(rope: KvRope) -> list:
    out = (ctypes.c_double * 64)()
    _check(lib().kv_rope_inv_freq(ctypes.byref(rope), out), "kv_rope_inv_freq")
    return list(out)


class RefStore:
    """Reference store of a row (see kv_ref_store): keys [L][slots][Hkv][128] bf16 and
    positions [slots] int32 (KV_REF_NONE = empty), both device tensors."""

    def __init__(self, k, pos):
        assert k.dim() == 4 and k.shape[3] == 128 and k.dtype == torch.bfloat16 and k.is_contiguous()
        assert pos.dtype == torch.int32 and pos.numel() == k.shape[1]
        self.k, self.pos = k, pos

    @classmethod
    def empty(cls, n_layers, n_slots, n_kv_heads, device):
        return cls(torch.zeros((n_layers, n_slots, n_kv_heads, 128), dtype=torch.bfloat16, device=device),
                   torch.full((n_slots,), KV_REF_NONE, dtype=torch.int32, device=device))

    def desc(self) -> KvRefStore:
        return KvRefStore(_ptr(self.k), _ptr(self.pos), int(self.k.shape[1]),
                          int(self.k.shape[1] * self.k.shape[2] * 128))


def kv_ref_invalidate(ref: RefStore, first, count):
    _check(lib().kv_ref_invalidate(ctypes.byref(ref.desc()), int(first), int(count),
                                   _stream(ref.pos.device)), "kv_ref_invalidate")


def kv_compact_rerope(src: PagedCache, dst: PagedCache, keep_tokens, n_keep, max_keep, old_pos,
                      new_pos=None, renumber_base=-1, rope_theta=1e6, limit=0, meta=None, rope=None,
                      ref_src=None, ref_dst=None):
    """Gather + exact re-rotation (see kv_compact_rerope / kv_compact_rerope_ex); meta is a
    list of (src, dst) tensor pairs gathered with the keep list.  rope (a KvRope) replaces
    rope_theta; ref_src / ref_dst are RefStore objects."""
    arr, n_meta = _meta_array(meta)
    if rope is None and ref_src is None and ref_dst is None:
        _check(lib().kv_compact_rerope(ctypes.byref(src.desc()), ctypes.byref(dst.desc()),
                                       _ptr(keep_tokens), _ptr(n_keep), int(max_keep), _ptr(old_pos),
                                       _ptr(new_pos), int(renumber_base), float(rope_theta), int(limit),
                                       arr, n_meta, _stream(src.k.device)), "kv_compact_rerope")
        return
    rope = rope if rope is not None else kv_rope("default", base=rope_theta)
    rs = ctypes.byref(ref_src.desc()) if ref_src is not None else None
    rd = ctypes.byref(ref_dst.desc()) if ref_dst is not None else None
    _check(lib().kv_compact_rerope_ex(ctypes.byref(src.desc()), ctypes.byref(dst.desc()),
                                      _ptr(keep_tokens), _ptr(n_keep), int(max_keep), _ptr(old_pos),
                                      _ptr(new_pos), int(renumber_base), ctypes.byref(rope), int(limit),
                                      arr, n_meta, rs, rd, _stream(src.k.device)), "kv_compact_rerope_ex")


def kv_compact_segment_remap(cache: PagedCache, prefix_len, evict_len, block_table_out, old_pos, new_pos,
                             freed_pages=None, renumber_base=-1, rope_theta=1e6, limit=0, meta=None, rope=None):
    """Page-table segment eviction (see kv_compact_segment_remap): the suffix is relinked
    in block_table_out, keys whose position changes are re-rotated in place; meta is a
    list of (src, dst) tensor pairs indexed by logical token."""
    if cache.block_table is None:
        raise ValueError("kv_compact_segment_remap needs a paged cache with a block table")
    rope = rope if rope is not None else kv_rope("default", base=rope_theta)
    arr, n_meta = _meta_array(meta or [])
    _check(lib().kv_compact_segment_remap(ctypes.byref(cache.desc()), int(prefix_len), int(evict_len),
                                          _ptr(block_table_out), _ptr(freed_pages), _ptr(old_pos), _ptr(new_pos),
                                          int(renumber_base), ctypes.byref(rope), int(limit), arr, n_meta,
                                          _stream(cache.k.device)),
           "kv_compact_segment_remap")


def kv_compact_pages_remap(cache: PagedCache, keep, n_keep, max_keep, block_table_out, old_pos, new_pos,
                           renumber_base=-1, rope_theta=1e6, limit=0, meta=None, rope=None, status=None):
    """Page-table compaction of a page-mode selection (see kv_compact_pages_remap): the kept
    pages relinked in block_table_out, keys whose position changes re-rotated in place;
    meta is a list of (src, dst) tensor pairs; status (int32 device word) gets
    KV_STATUS_NOT_WHOLE_PAGES when the keep list is not whole pages."""
    if cache.block_table is None:
        raise ValueError("kv_compact_pages_remap needs a paged cache with a block table")
    rope = rope if rope is not None else kv_rope("default", base=rope_theta)
    arr, n_meta = _meta_array(meta or [])
    _check(lib().kv_compact_pages_remap(ctypes.byref(cache.desc()), _ptr(keep), _ptr(n_keep), int(max_keep),
                                        _ptr(block_table_out), _ptr(old_pos), _ptr(new_pos), int(renumber_base),
                                        ctypes.byref(rope), int(limit), arr, n_meta, _ptr(status),
                                        _stream(cache.k.device)),
           "kv_compact_pages_remap")


def kv_compact_segment_inplace(cache: PagedCache, prefix_len, evict_len, pos, renumber_base=-1,
                               rope_theta=1e6, limit=0, meta=None, rope=None, ref=None):
    """In-place segment eviction (see kv_compact_segment_inplace / _ex); meta is a list of
    tensors moved in place; ref is a RefStore moved in place."""
    arr, n_meta = _meta_array([(m, m) for m in (meta or [])])
    if rope is None and ref is None:
        _check(lib().kv_compact_segment_inplace(ctypes.byref(cache.desc()), int(prefix_len), int(evict_len),
                                                _ptr(pos), int(renumber_base), float(rope_theta), int(limit),
                                                arr, n_meta, _stream(cache.k.device)),
               "kv_compact_segment_inplace")
        return
    rope = rope if rope is not None else kv_rope("default", base=rope_theta)
    rf = ctypes.byref(ref.desc()) if ref is not None else None
    _check(lib().kv_compact_segment_inplace_ex(ctypes.byref(cache.desc()), int(prefix_len), int(evict_len),
                                               _ptr(pos), int(renumber_base), ctypes.byref(rope), int(limit),
                                               arr, n_meta, rf, _stream(cache.k.device)),
           "kv_compact_segment_inplace_ex")
