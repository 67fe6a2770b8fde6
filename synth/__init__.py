"""Seeded synthetic inputs for the KV scoring / selection / compaction path.

This module only draws random numbers and lays them out in the shapes of the pages'
workloads.  It holds none of the method's arithmetic (no attention, no scores, no
selection, no rotation), so both the HIP path and the CPU oracle can consume it.  The
per-span foresight bonus it draws stands in for the output of PACE's planner, which sits
above the path: both sides take it as input.

Workload shapes (from the pages; the value distributions are those of the generators below):
  * KV footprint of Qwen3-8B: 36 layers x 8 KV heads x 128 dims x (K,V) x bf16 =
    144 KiB per token (PACE, Sec. 1).
  * Qwen2.5-1.5B head shape 12 Q / 2 KV heads (MemDecay's models).
  * Mistral-7B shape 32 layers, 32 Q / 8 KV heads, RoPE base 1e4 (PACE's second model).
  * Budget 2,048 with 4 sinks and 128 recent (PACE, Table 1); 7 region labels
    (MemDecay, Method); page/block size 16 (ActKV, Table 1).
Every tensor kind draws from its own seeded stream, so changing one recipe does not
shift the others.
"""
from __future__ import annotations

import dataclasses
import math

import torch

N_REGIONS = 7
REGION_SYSTEM = 0  # label order: system, plan, user, tool_in, tool_out, retrieval, scratchpad

# stream ids for the per-kind generators
_S_K, _S_V, _S_Q, _S_REG, _S_RPAR, _S_STATE, _S_SPAN, _S_BT, _S_SCORE, _S_PLANT = range(10)


@dataclasses.dataclass
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    window: int
    page_size: int
    rope_theta: float
    policy: str            # "memdecay" | "h2o" | "segment"
    item_tokens: int       # 1 = token items, page_size = page items
    budget_tokens: int
    system_prefix: int = 0
    n_sink: int = 0
    n_recent: int = 0
    n_spans: int = 0
    renumber: bool = False
    limit: int = 0
    segment_prefix: int = 0
    segment_frac: float = 0.0
    rho: float = 0.9
    alpha: float = 1.0
    tau: float = 0.01
    dt_steps: int = 1
    span_len_min: int = 8
    span_len_max: int = 64
    region_span_log_uniform: bool = False

    @property
    def n_pages(self):
        return -(-self.n_tokens // self.page_size)

    @property
    def budget_items(self):
        return self.budget_tokens // self.item_tokens

    @property
    def kv_bytes_per_token(self):
        return self.n_layers * self.n_kv_heads * self.head_dim * 2 * 2


WORKLOADS = {w.name: w for w in (
    Workload("qwen2.5-1.5b-1layer-n512", 1, 12, 2, 128, 512, 32, 16, 1e6,
             "memdecay", 16, 128, system_prefix=32),
    Workload("qwen2.5-1.5b-n2048", 28, 12, 2, 128, 2048, 64, 16, 1e6,
             "memdecay", 16, 512, system_prefix=128),
    Workload("qwen3-8b-n100k", 36, 32, 8, 128, 100_000, 64, 16, 1e6,
             "h2o", 1, 2048, n_sink=4, n_recent=128, n_spans=200,
             renumber=True, limit=8192),
    Workload("mistral-7b-n131072-segment", 32, 32, 8, 128, 131_072, 0, 16, 1e4,
             "segment", 1, 0, segment_prefix=16_384, segment_frac=0.3,
             renumber=True),
    Workload("qwen3-8b-n1m", 36, 32, 8, 128, 1_000_000, 64, 16, 1e6,
             "memdecay", 16, 2048, system_prefix=128, n_sink=4, n_recent=128,
             n_spans=200, renumber=True, limit=8192,
             region_span_log_uniform=True, span_len_min=64, span_len_max=4096),
)}


def workload(name: str, **override) -> Workload:
    """A workload by its name (model shape, token count); keyword overrides shrink it for tests."""
    if name not in WORKLOADS:
        raise ValueError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return dataclasses.replace(WORKLOADS[name], **override)


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream * 7_919 + 17)
    return g


def _randn_bf16(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def kv_cache(w: Workload, seed=0, device="cpu", paged_shuffle=False, extra_pages=0, progress=None):
    """Paged K and V, [layers][physical pages][page][kv heads][head_dim] bf16 ~ N(0,1).

    With ``paged_shuffle`` the logical pages map to a random permutation of
    ``n_pages + extra_pages`` physical pages through an int32 block table; otherwise the
    block table is None (physical page = logical page).  Large caches are generated one
    layer at a time on ``device`` to bound temporary memory.
    """
    n_phys = w.n_pages + extra_pages
    shape = (w.n_layers, n_phys, w.page_size, w.n_kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.bfloat16, device=device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    gk, gv = _gen(seed, _S_K, device), _gen(seed, _S_V, device)
    for layer in range(w.n_layers):
        k[layer] = _randn_bf16(shape[1:], gk, device)
        v[layer] = _randn_bf16(shape[1:], gv, device)
        if progress is not None:
            progress(layer)
    bt = None
    if paged_shuffle:
        gb = _gen(seed, _S_BT, "cpu")
        bt = torch.randperm(n_phys, generator=gb)[: w.n_pages].to(torch.int32).to(device)
    return k, v, bt


def plant_heavy_keys(w: Workload, k, q, block_table=None, n_plant=8, gain=3.0, seed=0):
    """Copy scaled window-query directions into a few random key slots (all layers and
    KV heads) so that attention concentrates there and decay clocks reset.
    Returns the logical indices that were planted."""
    g = _gen(seed, _S_PLANT, "cpu")
    idx = torch.randperm(max(1, w.n_tokens - w.window), generator=g)[:n_plant]
    group = w.n_q_heads // w.n_kv_heads
    for j in idx.tolist():
        page, slot = divmod(j, w.page_size)
        phys = page if block_table is None else int(block_table[page])
        for kvh in range(w.n_kv_heads):
            src = q[:, -1, kvh * group, :].float() * gain
            k[:, phys, slot, kvh, :] = src.to(torch.bfloat16).to(k.device)
    return sorted(idx.tolist())


def window_queries(w: Workload, seed=0, device="cpu"):
    """Window queries [layers][W][Hq][D] bf16 ~ N(0,1) (already at their positions)."""
    g = _gen(seed, _S_Q, device)
    return _randn_bf16((w.n_layers, w.window, w.n_q_heads, w.head_dim), g, device)


def _span_lengths(n, lo, hi, log_uniform, gen):
    out = []
    total = 0
    while total < n:
        if log_uniform:
            u = torch.rand((), generator=gen).item()
            length = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        else:
            length = int(torch.randint(lo, hi + 1, (), generator=gen).item())
        length = min(length, n - total)
        out.append(length)
        total += length
    return out


def regions(w: Workload, seed=0):
    """Region label per token (uint8, CPU): the system prompt first, then contiguous
    spans of random length whose labels are drawn from the six non-system regions."""
    g = _gen(seed, _S_REG, "cpu")
    n = w.n_tokens
    reg = torch.empty(n, dtype=torch.uint8)
    reg[: w.system_prefix] = REGION_SYSTEM
    pos = w.system_prefix
    for length in _span_lengths(n - pos, w.span_len_min, w.span_len_max,
                                w.region_span_log_uniform, g):
        reg[pos:pos + length] = int(torch.randint(1, N_REGIONS, (), generator=g).item())
        pos += length
    return reg


def region_params(seed=0):
    """Per-region base priority b_r ~ U[0,2] and decay rate lambda_r ~ U[0.004, 0.05]
    (float32, CPU).  The lambda range spans the half-lives MemDecay measures."""
    g = _gen(seed, _S_RPAR, "cpu")
    b = torch.rand(N_REGIONS, generator=g) * 2.0
    lam = 0.004 + torch.rand(N_REGIONS, generator=g) * (0.05 - 0.004)
    return b.float(), lam.float()


def memdecay_state(w: Workload, seed=0):
    """Prior EWMA a ~ U[0, 2/N] (float32) and decay clock dt ~ U{0..min(age, 400)}
    (int32), where a token's age is the number of tokens after it."""
    g = _gen(seed, _S_STATE, "cpu")
    n = w.n_tokens
    a = torch.rand(n, generator=g) * (2.0 / n)
    age = torch.arange(n - 1, -1, -1)
    cap = torch.clamp(age, max=400) + 1
    dt = (torch.rand(n, generator=g) * cap).floor().to(torch.int32)
    return a.float(), dt


def h2o_state(w: Workload, seed=0):
    """Prior accumulated attention ~ U[0, 4] per token (float32)."""
    g = _gen(seed, _S_STATE, "cpu")
    return (torch.rand(w.n_tokens, generator=g) * 4.0).float()


def spans(w: Workload, seed=0, n_steps=16, p_needed=0.01, floor=50000.0):
    """Spans and the planner's per-span foresight bonus (PACE Sec. 3.1 and 7).

    ``n_spans`` spans partition the tokens with Dirichlet(1) lengths; each span is read
    by a future step with probability ``p_needed``, at a distance d ~ U{1..n_steps}.
    The planner that turns this table into bonuses sits above the scoring path, and the
    pages fix only the bonus's properties: it outranks attention scores, the soonest
    needed span ranks first, and it has a constant floor of 50K.  This stand-in for the
    planner's output gives a span read d steps ahead floor * (1 + 1/d) and a span that
    no future step reads 0.  Returns (span_id[N] int32, span_bonus[S] float32)."""
    g = _gen(seed, _S_SPAN, "cpu")
    s = w.n_spans
    n = w.n_tokens
    e = -torch.log(torch.rand(s, generator=g, dtype=torch.float64))
    frac = e / e.sum()
    bounds = torch.round(torch.cumsum(frac, 0) * n).to(torch.int64)
    bounds[-1] = n
    span_id = torch.empty(n, dtype=torch.int32)
    start = 0
    for i, end in enumerate(bounds.tolist()):
        span_id[start:end] = i
        start = max(start, end)
    needed = torch.rand(s, generator=g) < p_needed
    dist = torch.randint(1, n_steps + 1, (s,), generator=g)
    bonus = floor * (1.0 + 1.0 / dist.to(torch.float64))
    span_bonus = torch.where(needed, bonus, torch.zeros_like(bonus)).to(torch.float32)
    return span_id, span_bonus


def scores(n, seed=0, alphabet=None, nan_frac=0.0, neg_zero=False):
    """Item scores for selection tests (float32, CPU): N(0,1), or drawn from a small
    ``alphabet`` to force exact ties, optionally with NaNs and -0.0."""
    g = _gen(seed, _S_SCORE, "cpu")
    if alphabet is not None:
        a = torch.tensor(alphabet, dtype=torch.float32)
        s = a[torch.randint(0, len(alphabet), (n,), generator=g)]
    else:
        s = torch.randn(n, generator=g)
    if neg_zero:
        z = torch.rand(n, generator=g) < 0.1
        s = torch.where(z, torch.full_like(s, -0.0), s)
    if nan_frac > 0:
        m = torch.rand(n, generator=g) < nan_frac
        s = torch.where(m, torch.full_like(s, float("nan")), s)
    return s.float()


def pinned_mask(n, seed=0, frac=0.05):
    g = _gen(seed, _S_SCORE + 100, "cpu")
    return (torch.rand(n, generator=g) < frac).to(torch.uint8)
