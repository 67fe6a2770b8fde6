"""Plain CPU oracle for the KV-cache scoring / selection / compaction / re-RoPE path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module.  Only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call it.  It shares no code with the HIP path: it is written from the
four pages on agent-session KV eviction and from plain mathematics, in NumPy float64,
slowly and without blocking, fusion or reordering beyond what each definition states.

Pages and the parts used (cited by title and section):
  * "PACE: Keeping the Right Tokens in the KV Cache Is Not Enough for Long-Horizon
    LLM Agents" -- Sec. 2 (budgeted eviction, H2O / SnapKV / StreamingLLM),
    Sec. 3.1 (blueprint, foresight bonus), Sec. 3.2 (bounded positions, renumbering,
    Proposition 1, choosing the limit, non-compounding re-rotation through a reference
    store), Sec. 3.4 (evicted rows offloaded at every compaction), Sec. 3.5 (split-half
    RoPE, static frequency scaling), Table 1 (budget 2,048 incl. 4 sinks and 128
    recent), Sec. 7 (the bonus is added to the eviction score).
  * "MemDecay: Region-Aware KV Cache Eviction for Efficient LLM Agent Inference" --
    Method (region labels, EWMA, decay clock, composite score, pinned regions,
    page-mean eviction, half-life).
  * "Rethinking KV Cache Eviction for Agentic LLM Serving" (Penelope) -- the
    illustrative cost example, the single-request measurement, and Part one (free
    only the needed leading blocks of the private history).
  * "ActKV: Efficient LLM Agents through Action-Guided KV Cache Management" --
    Sec. 2.3 (attention score), Sec. 2.5 (paged KV layout and slot-map example),
    Sec. 3.3 (the three primitives), Sec. 5.1 and Algorithm 1 (LRFU keep scores, top-p
    hit mask), Sec. 7.1 and Algorithm 3 (score recovery from the LSE, maximum over the
    GQA group), Sec. 7.2 and Algorithm 4 (in-place tail compaction).

Readings of points the pages leave open are listed next to each function.
Parity status: every function here is pinned by a ``-m "not gpu"`` test.  The foresight
bonus values themselves come from PACE's planner, which sits above this path: the
oracle takes them as an input (one value per span) exactly as the library does.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 rounding (storage type of cached keys and values)
# --------------------------------------------------------------------------------------

BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bf16


def bf16_round(x):
    """Round float64 values to the nearest bf16 value, ties to even (RNE).

    bf16 keeps 8 significant bits, the float32 exponent range, and subnormals down to
    2**-133.  For |x| in [2**(e-1), 2**e) the spacing is 2**(e-8); below the smallest
    normal 2**-126 the spacing stays 2**-133.  Scaling by a power of two is exact, so
    ``rint`` (round half to even) on the scaled value is exact RNE.
    Returns float64 arrays holding exactly representable bf16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e, -125) - 8
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits(x):
    """uint16 bit patterns of float64 values that are exactly bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """float64 values of uint16 bf16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# Paged KV layout (ActKV Sec. 2.5)
# --------------------------------------------------------------------------------------

def slot_map(block_table, page_size, n_tokens):
    """Physical slot of each logical token: block_table[j // BS] * BS + j % BS.

    ActKV Sec. 2.5: a block table maps logical token positions to physical blocks of
    BS slots; with BS=2, block_table=[17, 9] and 3 used tokens the slots are
    [34, 35, 18].
    """
    bt = np.asarray(block_table, dtype=np.int64)
    return [int(bt[j // page_size]) * page_size + j % page_size for j in range(n_tokens)]


def gather_logical(paged, block_table, page_size, n_tokens):
    """Logical-order view of one paged cache tensor.

    ``paged`` is [layers][physical_pages][page_size][kv_heads][head_dim] (ActKV's
    PagedKVCache[.., B, BS, H, D] per layer); returns [layers][n_tokens][kv_heads][D].
    ``block_table=None`` means physical page == logical page.
    """
    paged = np.asarray(paged)
    nl, npg, ps, hk, d = paged.shape
    assert ps == page_size
    flat = paged.reshape(nl, npg * ps, hk, d)
    if block_table is None:
        slots = np.arange(n_tokens)
    else:
        slots = np.asarray(slot_map(block_table, page_size, n_tokens), dtype=np.int64)
    return flat[:, slots]


# --------------------------------------------------------------------------------------
# O1: windowed attention mass  (MemDecay Method; ActKV Sec. 2.3 and 7.1; PACE Sec. 2)
# --------------------------------------------------------------------------------------

def attention_mass(q, k, scale=None, lse=None):
    """Windowed softmax attention mass received by every cached token.

    q: [L][W][Hq][D] window queries (already rotated at their own positions),
    k: [L][N][Hkv][D] cached keys in logical order.  Returns (mass[N], lse[L][Hq][W]).
    lse: optional [L][Hq][W] natural-log LSE supplied by the attention backend (ActKV
    Sec. 7.1 recovers A from it); computed from the keys when None.

    For layer l, query head h (KV head g = h // (Hq/Hkv), contiguous GQA groups) and
    window query w, which sits at logical position N - W + w and sees keys j <= N-W+w:
        s_j  = scale * <q[l,w,h], k[l,j,g]>
        LSE  = log sum_j exp(s_j)                 (ActKV Sec. 7.1's log-sum-exp)
        A_j  = exp(s_j - LSE)                     (softmax, ActKV Sec. 2.3)
        mass_j = sum over (l, h, w) of A_j        (masked keys contribute 0)
    Readings: scale defaults to 1/sqrt(D) (ActKV prints softmax(q K^T) without a scale;
    the standard attention scale is used); the window's own keys are scored causally.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nl, w_len, hq, d = q.shape
    nl2, n, hkv, d2 = k.shape
    assert nl == nl2 and d == d2 and hq % hkv == 0 and 1 <= w_len <= n
    g_size = hq // hkv
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    qpos = n - w_len + np.arange(w_len)
    visible = np.arange(n)[None, :] <= qpos[:, None]          # [W][N]
    mass = np.zeros(n, dtype=np.float64)
    lse_out = np.zeros((nl, hq, w_len), dtype=np.float64)
    for layer in range(nl):
        for h in range(hq):
            g = h // g_size
            s = scale * (q[layer, :, h, :] @ k[layer, :, g, :].T)   # [W][N]
            s = np.where(visible, s, -np.inf)
            if lse is None:
                m = s.max(axis=1, keepdims=True)
                row_lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            else:
                row_lse = np.asarray(lse, dtype=np.float64)[layer, h]
            a = np.exp(s - row_lse[:, None])                       # 0 where masked
            mass += a.sum(axis=0)
            lse_out[layer, h] = row_lse
    return mass, lse_out


def attention_score_max_group(q, k, scale=None, lse=None):
    """Attention score with the maximum over each GQA group (ActKV Sec. 7.1, Algorithm 3).

    q: [L][W][Hq][D], k: [L][N][Hkv][D] as in attention_mass.  For layer l, KV head g and
    window (action) query w, a key's attention is the maximum over the query heads h of
    g's group of A_j = exp(s_j - LSE) (same s, LSE and causal visibility as
    attention_mass).  ActKV keeps a running mean of it over the action queries; the score
    here sums it over window queries, KV heads and layers (one keep list serves every
    layer and head), so that score / (L*Hkv*W) is the mean.
    lse: optional [L][Hq][W] natural-log LSE supplied by the attention backend (ActKV
    recovers scores from it); computed from the keys when None.
    Returns (score[N], lse[L][Hq][W]).
    Reading: ActKV does not say how the per-(layer, KV head) scores combine into one keep
    mask; summing them follows MemDecay's mean over layers and heads.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nl, w_len, hq, d = q.shape
    nl2, n, hkv, d2 = k.shape
    assert nl == nl2 and d == d2 and hq % hkv == 0 and 1 <= w_len <= n
    g_size = hq // hkv
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    qpos = n - w_len + np.arange(w_len)
    visible = np.arange(n)[None, :] <= qpos[:, None]          # [W][N]
    score = np.zeros(n, dtype=np.float64)
    lse_out = np.zeros((nl, hq, w_len), dtype=np.float64)
    for layer in range(nl):
        for g in range(hkv):
            best = np.zeros((w_len, n), dtype=np.float64)       # max over the group
            for h in range(g * g_size, (g + 1) * g_size):
                s = scale * (q[layer, :, h, :] @ k[layer, :, g, :].T)
                s = np.where(visible, s, -np.inf)
                if lse is None:
                    m = s.max(axis=1, keepdims=True)
                    row_lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
                else:
                    row_lse = np.asarray(lse, dtype=np.float64)[layer, h]
                lse_out[layer, h] = row_lse
                best = np.maximum(best, np.exp(s - row_lse[:, None]))
            score += best.sum(axis=0)
    return score, lse_out


# --------------------------------------------------------------------------------------
# O3: foresight bonus of each token  (PACE Sec. 3.1 and Sec. 7)
# --------------------------------------------------------------------------------------

def token_bonus(span_id, span_bonus):
    """Bonus of each token: the bonus of the span it belongs to.  PACE's planner turns its
    forward-reference table into one bonus per span (Sec. 3.1) and the bonus is added to
    the eviction score (Sec. 7); the per-span values are its output and arrive here as
    ``span_bonus``.  A token outside every span (id -1) gets none.  Reading: an id that
    names no span of the table (negative, or not below the number of spans) is treated
    the same way, as no span."""
    sid = np.asarray(span_id, dtype=np.int64)
    sb = np.asarray(span_bonus, dtype=np.float64)
    out = np.zeros(sid.shape, dtype=np.float64)
    for i, s in enumerate(sid.tolist()):
        if 0 <= s < len(sb):
            out[i] = sb[s]
    return out


# --------------------------------------------------------------------------------------
# O2: MemDecay and H2O epilogues
# --------------------------------------------------------------------------------------

def memdecay_update(abar, region, base_prio, decay_rate, rho, alpha, tau, dt_steps,
                    ewma, clock, bonus=None):
    """One MemDecay scoring step (MemDecay, Method).

        a_i  <- rho * a_i + (1 - rho) * Abar_i
        dt_i <- 0 if Abar_i > tau else dt_i + dt_steps        (clock resets on use)
        s_i   = b_r(i) * exp(-lambda_r(i) * dt_i) + alpha * a_i  (+ foresight bonus)
    Readings: updates in the order EWMA, clock, score; "attention above tau" is a
    strict comparison of the windowed Abar_i; dt counts decode steps, dt_steps per
    observation (k > 1 for sampled intervals).  A label outside the region table names
    no region: its b and lambda are taken as 0 (the library also reports it in a status
    bit).  Returns (ewma', clock', score).
    """
    abar = np.asarray(abar, dtype=np.float64)
    r = np.asarray(region, dtype=np.int64)
    bp = np.asarray(base_prio, dtype=np.float64)
    dr = np.asarray(decay_rate, dtype=np.float64)
    known = (r >= 0) & (r < len(bp))
    b = np.where(known, bp[np.where(known, r, 0)], 0.0)
    lam = np.where(known, dr[np.where(known, r, 0)], 0.0)
    a_new = rho * np.asarray(ewma, dtype=np.float64) + (1.0 - rho) * abar
    clock = np.asarray(clock, dtype=np.int64)
    c_new = np.where(abar > tau, 0, clock + dt_steps)
    s = b * np.exp(-lam * c_new) + alpha * a_new
    if bonus is not None:
        s = s + np.asarray(bonus, dtype=np.float64)
    return a_new, c_new, s


def h2o_update(mass, accum, bonus=None):
    """H2O accumulated attention (PACE Sec. 2): acc <- acc + mass; s = acc (+ bonus)."""
    acc = np.asarray(accum, dtype=np.float64) + np.asarray(mass, dtype=np.float64)
    s = acc.copy()
    if bonus is not None:
        s = s + np.asarray(bonus, dtype=np.float64)
    return acc, s


def pinned_tokens(n_tokens, region=None, pinned_regions=0, n_sink=0, n_recent=0,
                  token_pinned=None, n_regions=32):
    """Tokens kept unconditionally.

    MemDecay pins whole regions (system by default); PACE's budget always includes 4
    sink and 128 recent tokens (Table 1).  A token is pinned if any rule pins it.
    ``pinned_regions`` is a bit mask over region labels; a label at or above n_regions
    names no region and pins nothing.
    """
    p = np.zeros(n_tokens, dtype=bool)
    if region is not None and pinned_regions:
        for i, r in enumerate(np.asarray(region, dtype=np.int64).tolist()):
            if 0 <= r < n_regions and (pinned_regions >> r) & 1:
                p[i] = True
    p[: min(n_sink, n_tokens)] = True
    if n_recent > 0:
        p[max(0, n_tokens - n_recent):] = True
    if token_pinned is not None:
        p |= np.asarray(token_pinned).astype(bool)
    return p


def page_mean(score, page_size):
    """MemDecay's page score S_p = (1/|p|) sum_{i in p} s_i over the tokens present."""
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    n_pages = -(-n // page_size)
    return np.array([s[p * page_size:min(n, (p + 1) * page_size)].mean()
                     for p in range(n_pages)])


def page_any(flags, page_size):
    """A page is pinned when any of its tokens is pinned (keeps pinned tokens alive)."""
    f = np.asarray(flags).astype(bool)
    n = f.shape[0]
    n_pages = -(-n // page_size)
    return np.array([f[p * page_size:min(n, (p + 1) * page_size)].any()
                     for p in range(n_pages)])


# --------------------------------------------------------------------------------------
# O4: budget selection (MemDecay Method; PACE Table 1; ActKV Sec. 3.3 "Eviction")
# --------------------------------------------------------------------------------------

STATUS_PINNED_OVER_BUDGET = 1
STATUS_NAN_SCORE = 2


def select_items(score, pinned, budget):
    """Keep all pinned items, then the best (budget - #pinned) others.

    Total order on items: higher score first; on an exact tie the lower index first;
    -0.0 counts as +0.0; NaN scores order after every number.  Returns
    (kept item indices ascending, status bits).  When the pinned items alone exceed
    the budget they are all kept (MemDecay keeps pinned tokens unconditionally) and
    STATUS_PINNED_OVER_BUDGET is set.
    """
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    pin = np.zeros(n, dtype=bool) if pinned is None else np.asarray(pinned).astype(bool)
    status = 0
    if np.isnan(s).any():
        status |= STATUS_NAN_SCORE
    pinned_idx = [i for i in range(n) if pin[i]]
    others = [i for i in range(n) if not pin[i]]

    def order_key(i):
        v = s[i]
        if math.isnan(v):
            return (1, 0.0, i)
        return (0, -(v + 0.0), i)

    others.sort(key=order_key)
    room = budget - len(pinned_idx)
    if room < 0:
        status |= STATUS_PINNED_OVER_BUDGET
        room = 0
    kept = sorted(pinned_idx + others[:room])
    return np.array(kept, dtype=np.int64), status


def expand_items(items, item_tokens, n_tokens):
    """Token indices of kept items, ascending; a partial last page keeps what it has."""
    out = []
    for it in items:
        for t in range(int(it) * item_tokens, min(n_tokens, (int(it) + 1) * item_tokens)):
            out.append(t)
    return np.array(out, dtype=np.int64)


# --------------------------------------------------------------------------------------
# O4b: ActKV LRFU keep scores with the top-p hit mask (ActKV Sec. 5.1, Algorithm 1)
# --------------------------------------------------------------------------------------

def exact_score_units(score):
    """Every float32 score as an exact integer multiple of 2**-149 (the spacing of the
    smallest float32 subnormal): a finite positive score s becomes the Python int s * 2**149,
    any other value (zero, negative, NaN, infinity) 0.  Sums of these integers are the exact
    sums of the scores, with no rounding anywhere."""
    sc = np.asarray(score, dtype=np.float32)
    out = []
    for x in sc.tolist():                        # float32 values as exact Python floats
        if math.isfinite(x) and x > 0.0:
            num, den = x.as_integer_ratio()      # den is a power of two <= 2**149
            out.append(num * ((1 << 149) // den))
        else:
            out.append(0)
    return out


def topp_hit_mask(score, p):
    """Hit mask of ActKV's LRFU (Sec. 5.1, Algorithm 1): an entry is a hit when its
    action-region score lies in the top-p set.

    Reading (a nucleus set): order the entries by score descending, exact ties by index
    ascending (-0 == +0); only finite positive scores carry weight, and their weight is
    the score itself, summed exactly (rational arithmetic, no rounding); the top-p set is
    the shortest prefix of that order whose weight reaches p times the total weight, p
    taken as the float32 the device receives.  Entries without weight are never hits, so
    p = 1 makes every positive score a hit, and p = 0 (or no positive score) none.
    """
    sc = np.asarray(score, dtype=np.float32)
    w = exact_score_units(sc)
    total = sum(w)
    target = Fraction(float(np.float32(p))) * total       # exact: p * (sum of the scores)
    hit = np.zeros(len(sc), dtype=bool)
    if target <= 0:
        return hit
    key = np.where(np.isnan(sc), -np.inf, sc.astype(np.float64))
    key = np.where(key == 0, 0.0, key)
    order = sorted(range(len(sc)), key=lambda j: (-key[j], j))
    acc = 0
    for j in order:
        if acc >= target or w[j] == 0:
            break
        hit[j] = True
        acc += w[j]
    return hit


def lrfu_update(keep_score, attn_score, p=0.9, decay=0.5):
    """One keep-score step of ActKV's attention-aware LRFU (Sec. 5.1, Algorithm 1):
    KS <- decay * KS + AttnScore on hits, KS <- decay * KS on misses.  New entries
    enter with KS = 0 (the caller appends zeros).  float64; returns (KS', hit)."""
    a = np.asarray(attn_score, dtype=np.float32)
    hit = topp_hit_mask(a, p)
    ks = float(np.float32(decay)) * np.asarray(keep_score, dtype=np.float64)
    ks = ks + np.where(hit, a.astype(np.float64), 0.0)
    return ks, hit


# --------------------------------------------------------------------------------------
# O4c: ActKV in-place tail compaction (ActKV Sec. 7.2, Algorithm 4)
# --------------------------------------------------------------------------------------

def tail_window(n_tokens, budget, block):
    """Target region of the compaction: the last X = ceil(budget/block) of the
    Y = ceil(n_tokens/block) logical blocks, from start = (Y - X)*block for budget
    slots.  Returns (start, end)."""
    y = -(-n_tokens // block)
    x = -(-budget // block)
    start = (y - x) * block
    return start, start + budget


def tail_compaction_pairs(n_tokens, keep, budget, block):
    """Copy plan of Algorithm 4: destinations are the slots of the target region whose
    entries are not kept, sources the kept entries outside it, both ascending, paired in
    order.  Sources and destinations are disjoint, so all copies can run at once.
    Returns (start, end, src, dst, overflow) with overflow when more kept entries lie
    outside the region than it has free slots (only the first ones are paired)."""
    start, end = tail_window(n_tokens, budget, block)
    keep = np.asarray(keep, dtype=np.int64)
    inside = set(int(j) for j in keep if start <= j < end)
    dst = [p for p in range(start, end) if p not in inside]
    src = [int(j) for j in keep if not (start <= j < end)]
    n = min(len(src), len(dst))
    return start, end, np.array(src[:n], dtype=np.int64), np.array(dst[:n], dtype=np.int64), len(src) > len(dst)


def tail_compact(arr, src, dst):
    """Apply the plan to a logical array [..., slots, ...] along axis 1 (slot axis):
    arr[:, dst] = arr[:, src].  Metadata arrays [slots] use axis 0 (pass arr[None])."""
    out = np.array(arr, copy=True)
    out[:, dst] = np.asarray(arr)[:, src]
    return out


# --------------------------------------------------------------------------------------
# O5: Penelope segment eviction and recompute cost
# --------------------------------------------------------------------------------------

def segment_evict_len(n_tokens, prefix_len, evict_tokens, block):
    """Tokens actually freed: the needed count rounded up to whole blocks, capped at
    the private history (Penelope, Part one: split at block boundaries and free only
    the leading blocks needed)."""
    e = -(-evict_tokens // block) * block
    return max(0, min(e, n_tokens - prefix_len))


def select_segment(n_tokens, prefix_len, evict_tokens, block):
    """Keep [0, P) and [P + E', N): delete from the front of the private history."""
    e = segment_evict_len(n_tokens, prefix_len, evict_tokens, block)
    keep = list(range(prefix_len)) + list(range(prefix_len + e, n_tokens))
    return np.array(keep, dtype=np.int64)


QWEN3_8B_LINEAR_UNITS = 23552


def recompute_cost(a, b, linear_units=QWEN3_8B_LINEAR_UNITS):
    """Cost of recomputing tokens at positions [a, b).

    Penelope's model: one unit is one query-key pair; a token at position p attends to
    the p tokens before it and its linear/FFN work is a position-independent constant
    (23,552 units for Qwen3-8B).  Summed one token at a time.
    """
    return float(sum(linear_units + p for p in range(a, b)))


# --------------------------------------------------------------------------------------
# O6: exact re-rotation and compaction  (PACE Sec. 3.2 Proposition 1, Sec. 3.5)
# --------------------------------------------------------------------------------------

def rope_inv_freq(theta, head_dim):
    """theta_i = base ** (-2 i / D), i < D/2 (standard RoPE frequencies), float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_rotate(k, delta, theta=None, inv_freq=None):
    """Rotate split-half RoPE pairs (i, i + D/2) of k[..., D] by angle delta * theta_i.

        x' = x cos(phi) - y sin(phi),   y' = x sin(phi) + y cos(phi)
    ``delta`` broadcasts against k's leading dims.  The frequencies are base ** (-2i/D)
    for a scalar ``theta``, or the given ``inv_freq`` table.  float64 throughout.
    """
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[-1]
    half = d // 2
    freq = rope_inv_freq(theta, d) if inv_freq is None else np.asarray(inv_freq, dtype=np.float64)
    assert freq.shape == (half,)
    phi = np.asarray(delta, dtype=np.float64)[..., None] * freq
    c, s = np.cos(phi), np.sin(phi)
    x, y = k[..., :half], k[..., half:]
    return np.concatenate([x * c - y * s, x * s + y * c], axis=-1)


def scaled_inv_freq(kind, base, head_dim=128, factor=1.0, original_max_position=8192,
                    low_freq_factor=1.0, high_freq_factor=4.0, beta_fast=32.0, beta_slow=1.0,
                    truncate=True):
    """RoPE frequencies under static scaling (PACE Sec. 3.5 names default, linear, YaRN
    and Llama-3 style scaling; the definitions are the published methods):
      default: theta_i = base ** (-2i/D);
      linear:  theta_i / factor (position interpolation);
      llama3:  wavelength w_i = 2 pi / theta_i.  Dims with w_i < L / high_freq_factor keep
               theta_i, dims with w_i > L / low_freq_factor get theta_i / factor, the rest
               blend (1 - t) theta_i / factor + t theta_i with
               t = (L / w_i - low_freq_factor) / (high_freq_factor - low_freq_factor);
      yarn:    "NTK-by-parts" as the YaRN authors' code and the inference engines build
               it: pair i turns r_i = L / w_i times over the original context L, and the
               pair index at which r_i equals beta turns is
                   i(beta) = D * ln(L / (2 pi beta)) / (2 ln base);
               with lo = i(beta_fast) and hi = i(beta_slow) (lo rounded down and hi up when
               truncate, then clamped to [0, D - 1]; hi = lo + 0.001 when they meet) the ramp
               g_i = clip((i - lo) / (hi - lo), 0, 1) runs over the pair index and
               theta'_i = g_i theta_i / factor + (1 - g_i) theta_i;
      yarn_ratio: the ramp written over r_i instead, as the YaRN paper states it:
               g = clip((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1),
               theta'_i = (1 - g) theta_i / factor + g theta_i.
    The two YaRN forms agree outside the blended band and differ inside it (r_i falls
    exponentially with i); keys cached by an engine carry the first.
    L = original_max_position.  Only the rotation is defined here: YaRN's attention
    temperature scales q and k when they are cached, and re-rotating a cached key by a
    position difference leaves that factor in place.
    """
    theta = rope_inv_freq(base, head_dim)
    if kind == "default":
        return theta
    if kind == "linear":
        return theta / factor
    wavelen = 2.0 * math.pi / theta
    L = float(original_max_position)
    if kind == "llama3":
        out = np.empty_like(theta)
        for i in range(theta.size):
            if wavelen[i] < L / high_freq_factor:
                out[i] = theta[i]
            elif wavelen[i] > L / low_freq_factor:
                out[i] = theta[i] / factor
            else:
                t = (L / wavelen[i] - low_freq_factor) / (high_freq_factor - low_freq_factor)
                out[i] = (1.0 - t) * theta[i] / factor + t * theta[i]
        return out
    if kind == "yarn":
        def pair_at(turns):
            return head_dim * math.log(L / (turns * 2.0 * math.pi)) / (2.0 * math.log(base))
        lo, hi = pair_at(beta_fast), pair_at(beta_slow)
        if truncate:
            lo, hi = math.floor(lo), math.ceil(hi)
        lo, hi = max(lo, 0), min(hi, head_dim - 1)
        if hi == lo:
            hi = hi + 0.001
        out = np.empty_like(theta)
        for i in range(theta.size):
            g = min(max((i - lo) / (hi - lo), 0.0), 1.0)
            out[i] = g * theta[i] / factor + (1.0 - g) * theta[i]
        return out
    if kind == "yarn_ratio":
        r = L / wavelen
        g = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
        return (1.0 - g) * theta / factor + g * theta
    raise ValueError(kind)


def renumbered_positions(n_keep, renumber_base, old_pos_kept):
    """New physical positions: base + rank when renumbering (order-preserving and
    gap-collapsing, PACE Sec. 3.2), otherwise unchanged."""
    if renumber_base is None or renumber_base < 0:
        return np.asarray(old_pos_kept, dtype=np.int64).copy()
    return renumber_base + np.arange(n_keep, dtype=np.int64)


def compact_rerope(k, v, keep, old_pos, renumber_base, theta, inv_freq=None):
    """Stable in-order gather of kept tokens plus exact re-rotation of their keys.

    k, v: [L][N][Hkv][D] logical arrays holding bf16 values; keep: ascending kept token
    indices.  Rank r takes source j = keep[r].  V is copied verbatim.  K is copied
    verbatim when delta = new_pos - old_pos is 0, otherwise rotated by delta in float64
    (Proposition 1: re-rotating the cached key by the position difference gives the key
    at the new position) and rounded once to bf16 (RNE).  The frequencies are
    theta ** (-2i/D), or the inv_freq table when given (scaled RoPE).
    Returns (k', v', new_pos).
    Reading: the "fp32" derivation of the pages is evaluated here in float64 from the
    exact bf16 inputs, so the oracle holds the correctly rounded result.
    """
    keep = np.asarray(keep, dtype=np.int64)
    old_kept = np.asarray(old_pos, dtype=np.int64)[keep]
    new_pos = renumbered_positions(len(keep), renumber_base, old_kept)
    delta = new_pos - old_kept
    kk = np.asarray(k, dtype=np.float64)[:, keep]
    vv = np.asarray(v, dtype=np.float64)[:, keep].copy()
    out_k = kk.copy()
    moved = np.nonzero(delta != 0)[0]
    if moved.size:
        rot = rope_rotate(kk[:, moved], delta[moved][None, :, None], theta, inv_freq)
        out_k[:, moved] = bf16_round(rot)
    return out_k, vv, new_pos


REF_NONE = -(2 ** 31)   # position of an empty reference-store entry


def compact_rerope_store(k, v, keep, old_pos, renumber_base, inv_freq, ref_k, ref_pos):
    """compact_rerope with PACE's reference store (Sec. 3.2, non-compounding re-rotation).

    ref_k: [L][N][Hkv][D] reference keys and ref_pos: [N] the position each is valid at
    (REF_NONE = empty), indexed by source token like k.  For rank r with source j, old
    position op and new position np:
      * the entry is used when it is not empty and the stored key, re-rotated from
        ref_pos[j] to op and rounded, equals the cached key bit for bit (the check
        against the stored key); the new key is then the stored key rotated by
        np - ref_pos[j] and rounded once, and the entry moves to slot r;
      * otherwise, when the position changes, this is the key's first re-rotation: the
        cached key and op are copied into the store at slot r and the new key is the
        cached key rotated by np - op, rounded once;
      * otherwise the key is copied and slot r of the store stays empty.
    Every key therefore carries at most two roundings: the engine's own when it cached
    the key, and one from the stored copy.  Returns (k', v', new_pos, ref_k', ref_pos',
    used) where ref_k' is defined where ref_pos' is not REF_NONE and used[r] says
    whether the store entry served rank r.
    Reading: entries are created at the first position change (a key that never moves
    has no rounding to protect against); PACE does not say more.
    """
    keep = np.asarray(keep, dtype=np.int64)
    k = np.asarray(k, dtype=np.float64)
    ref_k = np.asarray(ref_k, dtype=np.float64)
    ref_pos = np.asarray(ref_pos, dtype=np.int64)
    old_kept = np.asarray(old_pos, dtype=np.int64)[keep]
    new_pos = renumbered_positions(len(keep), renumber_base, old_kept)
    nl, _, hkv, d = k.shape
    out_k = np.zeros((nl, len(keep), hkv, d))
    out_ref = np.zeros((nl, len(keep), hkv, d))
    out_ref_pos = np.full(len(keep), REF_NONE, dtype=np.int64)
    used = np.zeros(len(keep), dtype=bool)
    for r, j in enumerate(keep):
        op, np_ = old_kept[r], new_pos[r]
        valid = False
        if ref_pos[j] != REF_NONE:
            back = bf16_round(rope_rotate(ref_k[:, j], op - ref_pos[j], inv_freq=inv_freq))
            valid = bool((back == k[:, j]).all())
        if valid:
            out_k[:, r] = bf16_round(rope_rotate(ref_k[:, j], np_ - ref_pos[j], inv_freq=inv_freq))
            out_ref[:, r] = ref_k[:, j]
            out_ref_pos[r] = ref_pos[j]
            used[r] = True
        elif np_ != op:
            out_k[:, r] = bf16_round(rope_rotate(k[:, j], np_ - op, inv_freq=inv_freq))
            out_ref[:, r] = k[:, j]
            out_ref_pos[r] = op
        else:
            out_k[:, r] = k[:, j]
    vv = np.asarray(v, dtype=np.float64)[:, keep].copy()
    return out_k, vv, new_pos, out_ref, out_ref_pos, used


def evicted_tokens(n_tokens, keep):
    """Tokens a compaction drops: the complement of the keep list in [0, N), ascending
    (PACE Sec. 3.4 offloads them to host memory at every compaction)."""
    mask = np.ones(n_tokens, dtype=bool)
    mask[np.asarray(keep, dtype=np.int64)] = False
    return np.nonzero(mask)[0]


def load_rows(dst, slots, rows):
    """Rows coming back from host memory: row r of ``rows`` ([L][count][Hkv][D]) lands in
    slot slots[r] of ``dst`` ([L][N][Hkv][D], logical order), every layer; other slots are
    unchanged.  Loading the rows a compaction dropped back into the slots they came from
    restores the row (the inverse of evicted-row offload, PACE Sec. 3.4; Penelope Part
    three moves segments back from the CPU tier)."""
    out = np.array(dst, copy=True)
    rows = np.asarray(rows)
    for r, j in enumerate(np.asarray(slots, dtype=np.int64).tolist()):
        out[:, j] = rows[:, r]
    return out


def chunked_swap(gpu, pool, slots, in_first, buf_first, chunk):
    """Penelope's swap when both tiers are full ("Rethinking KV Cache Eviction for Agentic
    LLM Serving", Part three): the segment held in GPU slots ``slots`` moves to the CPU,
    and the segment in CPU rows [in_first, in_first + count) moves into those GPU slots.
    Neither tier has free space, so a small CPU swap buffer (``chunk`` rows from buf_first,
    1,024 tokens in the paper) is used chunk by chunk:
      - the chunk leaving the GPU is written into the current buffer;
      - the GPU slots it freed receive the matching chunk coming from the CPU;
      - the CPU rows that chunk emptied become the buffer for the next chunk.
    gpu: [L][N][Hkv][D] logical rows; pool: [L][P][Hkv][D] CPU rows.
    Returns (gpu', pool', out_rows, next_buffer): out_rows[r] is the CPU row where the r-th
    outgoing row now lives, and next_buffer the first row of the CPU rows left free (the
    incoming segment's last chunk).
    Reading: chunks are taken in segment order and a chunk has the buffer's size except
    the last one."""
    gpu = np.array(gpu, copy=True)
    pool = np.array(pool, copy=True)
    slots = np.asarray(slots, dtype=np.int64)
    count = len(slots)
    assert buf_first + min(chunk, count) <= in_first or in_first + count <= buf_first
    buf = buf_first
    out_rows = []
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        leaving = slots[c0:c0 + n]
        pool[:, buf:buf + n] = gpu[:, leaving]
        out_rows.extend(range(buf, buf + n))
        gpu[:, leaving] = pool[:, in_first + c0:in_first + c0 + n]
        buf = in_first + c0
    return gpu, pool, np.array(out_rows, dtype=np.int64), buf


# --------------------------------------------------------------------------------------
# Renumber trigger and limit rule (PACE Sec. 3.2)
# --------------------------------------------------------------------------------------

def renumber_needed(next_pos, headroom, limit):
    """Renumber when the next physical position comes within the headroom of the limit.
    Reading: 'within h of L' means next_pos >= L - h."""
    return next_pos >= limit - headroom


def smallest_limit(budget, interval, chunk):
    """Smallest power-of-two limit with L >= R_max + C, R_max = budget + interval."""
    need = budget + interval + chunk
    limit = 1
    while limit < need:
        limit *= 2
    return limit


def simulate_renumbers(session_tokens, budget, limit, headroom):
    """Count renumbers in a session where eviction runs after every appended token.

    Tokens arrive one at a time; the resident row is evicted back to the budget; the
    trigger is checked after each eviction; a renumber moves the row to positions
    0..n-1 and the next token continues right after it (PACE Sec. 3.2).
    """
    next_pos = 0
    resident = 0
    count = 0
    for _ in range(session_tokens):
        next_pos += 1
        resident = min(resident + 1, budget)
        if renumber_needed(next_pos, headroom, limit):
            next_pos = resident
            count += 1
    return count


# --------------------------------------------------------------------------------------
# Whole pipeline on small inputs
# --------------------------------------------------------------------------------------

def score_step(q, k, *, policy, scale=None, region=None, base_prio=None, decay_rate=None,
               rho=0.9, alpha=1.0, tau=0.01, dt_steps=1, ewma=None, clock=None,
               accum=None, span_id=None, span_bonus=None,
               pinned_regions=0, n_sink=0, n_recent=0, token_pinned=None, item_tokens=1,
               aggregate="sum", lse_in=None):
    """Score one eviction step: mass -> policy epilogue -> per-item score and pin flag.

    aggregate 'sum' sums the attention over every query head (attention_mass);
    'max_group' takes the maximum over each GQA group first (attention_score_max_group,
    ActKV).  policy 'memdecay' divides by the number of summed terms, L*Hq*W or L*Hkv*W
    (the mean over layers, heads and window queries); policy 'h2o' accumulates the sum.  lse_in is an
    optional supplied LSE.  Returns a dict of float64 arrays.
    """
    nl, w_len, hq, _ = np.asarray(q).shape
    hkv = np.asarray(k).shape[2]
    if aggregate == "sum":
        mass, lse = attention_mass(q, k, scale, lse_in)
        terms = nl * hq * w_len
    elif aggregate == "max_group":
        mass, lse = attention_score_max_group(q, k, scale, lse_in)
        terms = nl * hkv * w_len
    else:
        raise ValueError(aggregate)
    n = mass.shape[0]
    bonus = None
    if span_id is not None and span_bonus is not None:
        bonus = token_bonus(span_id, span_bonus)
    out = {"mass": mass, "lse": lse}
    if policy == "memdecay":
        abar = mass / terms
        a, c, s = memdecay_update(abar, region, base_prio, decay_rate, rho, alpha, tau,
                                  dt_steps, ewma, clock, bonus)
        out.update(abar=abar, ewma=a, clock=c, token_score=s)
    elif policy == "h2o":
        acc, s = h2o_update(mass, accum if accum is not None else np.zeros(n), bonus)
        out.update(accum=acc, token_score=s)
    else:
        raise ValueError(policy)
    n_regions = len(base_prio) if base_prio is not None else 32
    pin = pinned_tokens(n, region, pinned_regions, n_sink, n_recent, token_pinned, n_regions)
    out["token_pinned"] = pin
    if item_tokens == 1:
        out["item_score"] = out["token_score"]
        out["item_pinned"] = pin
    else:
        out["item_score"] = page_mean(out["token_score"], item_tokens)
        out["item_pinned"] = page_any(pin, item_tokens)
    return out
