// C ABI of libkvscore: argument validation, workspace layout and launch order.
// The entry points and their contracts are documented in include/kvscore.h.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "kv_internal.h"

using namespace kvs;

namespace kvs {

bool trace_on() {
  static const bool on = [] {
    const char* v = getenv("KVSCORE_TRACE");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

void trace_launch(const char* fmt, ...) {
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[kvscore] %s\n", line);
}

}  // namespace kvs

namespace {

thread_local char g_err_text[512];

int32_t hip_fail(hipError_t e) {
  snprintf(g_err_text, sizeof(g_err_text), "HIP call failed: %s", hipGetErrorString(e));
  return KV_EHIP;
}

// gfx950 check, cached per device ordinal (immutable facts, safe to share).
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int32_t check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return KV_EUNSUPPORTED;
  int v = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    v = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? KV_OK : KV_EUNSUPPORTED;
}

// Scoring workgroups resident at once on an MI355X: two per CU (LDS-bound) x 256 CUs.
constexpr int64_t kResidentGroups = 512;
constexpr int64_t kCUs = 256;              // compute units of the part

int log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1LL << s) < v) ++s;
  return s;
}

int32_t check_cache(const kv_cache_desc* c) {
  if (!c || !c->k || !c->v) return KV_EINVAL;
  if (c->n_layers <= 0 || c->n_kv_heads <= 0 || c->n_tokens <= 0) return KV_EINVAL;
  if (c->n_tokens > 0x7FFFFFFFLL) return KV_EINVAL;
  if (c->head_dim != kHeadDim) return KV_EUNSUPPORTED;
  const int ps = log2_exact(c->page_size);
  if (ps < 0 || ps > 10) return KV_EUNSUPPORTED;
  const int64_t slot = (int64_t)c->n_kv_heads * c->head_dim;
  if (c->page_stride < slot * c->page_size) return KV_EINVAL;
  if (c->page_stride > 0xFFFFFFFFLL) return KV_EUNSUPPORTED;  // page offsets use 32-bit products
  if (c->n_layers > 1 && c->layer_stride < c->page_stride) return KV_EINVAL;
  if (((uintptr_t)c->k | (uintptr_t)c->v) & 15) return KV_EINVAL;
  if ((c->page_stride | c->layer_stride) & 7) return KV_EINVAL;  // keep 16-byte alignment
  return KV_OK;
}

struct ScoreLayout {
  int rows, group, row_stride, max_log, n_chunks, chunk, n_rsplit;
  size_t off_lse_part, off_lse2, off_mass, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int32_t score_layout(const kv_cache_desc* c, const kv_score_params* p, ScoreLayout* L) {
  int32_t rc = check_cache(c);
  if (rc) return rc;
  if (!p) return KV_EINVAL;
  if (p->n_q_heads <= 0 || p->n_q_heads % c->n_kv_heads) return KV_EINVAL;
  if (p->window <= 0 || p->window > c->n_tokens) return KV_EINVAL;
  const int group = p->n_q_heads / c->n_kv_heads;
  // rows per window query: G, or G rounded up to a power of two for the group maximum
  int row_stride = group, max_log = 0;
  if (p->aggregate == KV_AGG_MAX_GROUP) {
    while ((1 << max_log) < group) ++max_log;
    if (max_log > 5) return KV_EUNSUPPORTED;
    row_stride = 1 << max_log;
  } else if (p->aggregate != KV_AGG_SUM) {
    return KV_EINVAL;
  }
  const int64_t rows = (int64_t)row_stride * p->window;
  if (rows > kMaxRows) return KV_EUNSUPPORTED;
  // chunk: a multiple of the 64-key tile, large enough to amortise the query load and
  // small enough that the grid fills the chip
  const int n_rsplit = (int)((rows + kRowsPerGroup - 1) / kRowsPerGroup);
  const int64_t units = (int64_t)c->n_layers * c->n_kv_heads;
  const int64_t per_chunk = units * n_rsplit;   // workgroups per key chunk
  const int64_t n = c->n_tokens;
  int64_t chunk = 4096;
  if (per_chunk * ((n + 4095) / 4096) >= 2048) {
    // Enough work to choose a chunk of 2,048-8,192 keys whose grid fills whole rounds of
    // the chip's resident workgroups, so that the last round does not run mostly empty:
    // the largest chunk that keeps 99% of the slots busy on average, else the best fill.
    double best = 0.0;
    for (int64_t nch = (n + 8191) / 8192; nch <= (n + 2047) / 2048; ++nch) {
      const int64_t ch = ((n + nch - 1) / nch + kTile - 1) / kTile * kTile;
      const int64_t wgs = per_chunk * ((n + ch - 1) / ch);
      if (wgs < 2048) continue;
      const int64_t rounds = (wgs + kResidentGroups - 1) / kResidentGroups;
      const double fill = (double)per_chunk * n / ((double)kResidentGroups * rounds * ch);
      if (fill > best) {
        best = fill;
        chunk = ch;
      }
      if (fill >= 0.99) break;
    }
  } else {
    // Less work: a few rounds of resident workgroups at most, where whole rounds and the
    // fixed cost of each workgroup decide.  Cost of a chunking, in tile times of a CU
    // that two workgroups share: rounds x (tiles per chunk + about 4 tiles of fixed cost:
    // query load, ring fill, partial stores); a grid of at most one workgroup per CU runs
    // each at about 0.6 of that per tile.  The cheapest chunking wins, the larger chunk
    // on a tie.  (Fitted to measured rows of 512 to 100,000 keys, 1 to 36 layers.)
    double best = 1e300;
    for (int64_t nch = (n + 8191) / 8192; nch <= (n + kTile - 1) / kTile; ++nch) {
      const int64_t ch = ((n + nch - 1) / nch + kTile - 1) / kTile * kTile;
      const int64_t wgs = per_chunk * ((n + ch - 1) / ch);
      const double per = (double)(ch / kTile) + 4.0;
      const double cost =
          wgs <= kCUs ? 0.6 * per : (double)((wgs + kResidentGroups - 1) / kResidentGroups) * per;
      if (cost < best - 1e-9) {
        best = cost;
        chunk = ch;
      }
    }
  }
  L->rows = (int)rows;
  L->n_rsplit = n_rsplit;
  L->group = group;
  L->row_stride = row_stride;
  L->max_log = max_log;
  L->chunk = (int)chunk;
  L->n_chunks = (int)((c->n_tokens + chunk - 1) / chunk);
  size_t off = 0;
  L->off_lse_part = off;
  off = align256(off + (size_t)units * L->n_chunks * rows * sizeof(float2));
  L->off_lse2 = off;
  off = align256(off + (size_t)units * rows * sizeof(float));
  L->off_mass = off;
  off = align256(off + (size_t)units * n_rsplit * c->n_tokens * sizeof(float));
  L->total = off;
  return KV_OK;
}

int32_t check_meta(const kv_meta_desc* meta, int32_t n_meta, MetaSet* out) {
  memset(out, 0, sizeof(*out));
  if (n_meta < 0 || n_meta > KV_MAX_META) return KV_EINVAL;
  if (n_meta > 0 && !meta) return KV_EINVAL;
  for (int i = 0; i < n_meta; ++i) {
    const int b = meta[i].elem_bytes;
    if (!meta[i].src || !meta[i].dst || (b != 1 && b != 2 && b != 4 && b != 8)) return KV_EINVAL;
    out->src[i] = meta[i].src;
    out->dst[i] = meta[i].dst;
    out->elem_bytes[i] = b;
  }
  out->n = n_meta;
  return KV_OK;
}

}  // namespace

extern "C" {

int32_t kv_abi_version(void) { return KV_ABI_VERSION; }

const char* kv_strerror(int32_t code) {
  switch (code) {
    case KV_OK:
      return "ok";
    case KV_EINVAL:
      return "invalid argument (null pointer, size, stride or shape)";
    case KV_EUNSUPPORTED:
      return "unsupported (head_dim != 128, page size not a power of two <= 1024, "
             "more than 512 rows per KV head, a GQA group above 32 heads with the group "
             "maximum, page items above 256 tokens, or not a gfx950 device)";
    case KV_EWORKSPACE:
      return "workspace too small";
    case KV_EHIP:
      return g_err_text[0] ? g_err_text : "HIP call failed";
    case KV_ELIMIT:
      return "renumbered row does not fit under the position limit";
    default:
      return "unknown kvscore status";
  }
}

int32_t kv_renumber_needed(int64_t next_pos, int32_t headroom, int32_t limit) {
  return next_pos >= (int64_t)limit - headroom ? 1 : 0;
}

int32_t kv_score_workspace_size(const kv_cache_desc* cache, const kv_score_params* p,
                                size_t* bytes) {
  if (!bytes) return KV_EINVAL;
  ScoreLayout L;
  const int32_t rc = score_layout(cache, p, &L);
  if (rc) return rc;
  *bytes = L.total;
  return KV_OK;
}

int32_t kv_score(const kv_cache_desc* c, const kv_score_params* p, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  ScoreLayout L;
  int32_t rc = score_layout(c, p, &L);
  if (rc) return rc;
  if (!p->q || !p->item_score || !p->item_pinned) return KV_EINVAL;
  if (p->item_tokens != 1 && p->item_tokens != c->page_size) return KV_EINVAL;
  const int item_shift = log2_exact(p->item_tokens);
  if (item_shift > 8) return KV_EUNSUPPORTED;
  if (p->policy == KV_POLICY_MEMDECAY) {
    if (!p->ewma || !p->clock || !p->region || !p->base_prio || !p->decay_rate) return KV_EINVAL;
    if (p->n_regions <= 0 || p->n_regions > 32) return KV_EINVAL;
  } else if (p->policy == KV_POLICY_H2O) {
    if (!p->accum) return KV_EINVAL;
  } else {
    return KV_EINVAL;
  }
  if (p->region && (p->n_regions <= 0 || p->n_regions > 32)) return KV_EINVAL;
  if (p->span_id && (!p->span_bonus || p->n_spans <= 0)) return KV_EINVAL;
  if (p->n_sink < 0 || p->n_recent < 0 || p->dt_steps < 0) return KV_EINVAL;
  if (!ws || ws_bytes < L.total) return KV_EWORKSPACE;
  if ((rc = check_device())) return rc;

  char* w = (char*)ws;
  const float scale = p->scale != 0.f ? p->scale : 1.0f / sqrtf((float)kHeadDim);
  const float c2 = (float)((double)scale * 1.4426950408889634);
  const int n_lg = c->n_layers * c->n_kv_heads;
  hipError_t e;

  ScoreArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.k = (const uint16_t*)c->k;
  sa.layer_stride = c->layer_stride;
  sa.page_stride = c->page_stride;
  sa.block_table = c->block_table;
  sa.n_layers = c->n_layers;
  sa.n_kv_heads = c->n_kv_heads;
  sa.page_shift = log2_exact(c->page_size);
  sa.n_tokens = c->n_tokens;
  sa.q = (const uint16_t*)p->q;
  sa.n_q_heads = p->n_q_heads;
  sa.window = p->window;
  sa.group = L.group;
  sa.rows = L.rows;
  sa.row_stride = L.row_stride;
  sa.max_log = L.max_log;
  sa.n_rsplit = L.n_rsplit;
  sa.c = c2;
  sa.chunk = L.chunk;
  sa.n_chunks = L.n_chunks;
  sa.lse_part = (float2*)(w + L.off_lse_part);
  sa.lse2 = (const float*)(w + L.off_lse2);
  sa.mass_part = (float*)(w + L.off_mass);

  hipEvent_t* ev = p->stage_events;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return hip_fail(e);
  if (!p->lse_in) {
    if ((e = launch_score_pass(sa, false, stream)) != hipSuccess) return hip_fail(e);
  }
  if ((e = mark(1)) != hipSuccess) return hip_fail(e);
  CombineArgs ca;
  ca.lse_part = sa.lse_part;
  ca.n_chunks = L.n_chunks;
  ca.rows = L.rows;
  ca.n_kv_heads = c->n_kv_heads;
  ca.n_q_heads = p->n_q_heads;
  ca.group = L.group;
  ca.window = p->window;
  ca.row_stride = L.row_stride;
  ca.n_lg = n_lg;
  ca.lse_in = p->lse_in;
  ca.lse2 = (float*)(w + L.off_lse2);
  ca.lse_out = p->lse;
  ca.status = p->status;
  // A pass-2 grid of at most one round of resident workgroups, over at most 16 chunks,
  // combines its rows' LSE in each workgroup, which saves the combine launch (measured:
  // 4-7 us on rows of 512-8,000 keys; with 32 chunks per row the repeated combine cost
  // more than the launch).  Larger grids combine once per row in their own launch.
  sa.fuse_combine = (int64_t)n_lg * L.n_rsplit * L.n_chunks <= kResidentGroups && L.n_chunks <= 16 ? 1 : 0;
  sa.comb = ca;
  if (!sa.fuse_combine && (e = launch_lse_combine(ca, stream)) != hipSuccess) return hip_fail(e);
  if ((e = mark(2)) != hipSuccess) return hip_fail(e);
  if ((e = launch_score_pass(sa, true, stream)) != hipSuccess) return hip_fail(e);
  if ((e = mark(3)) != hipSuccess) return hip_fail(e);

  EpilogueArgs ea;
  memset(&ea, 0, sizeof(ea));
  ea.mass_part = sa.mass_part;
  ea.n_parts = n_lg * L.n_rsplit;
  ea.n_tokens = c->n_tokens;
  // MemDecay's mean over layers and heads: Hq terms per (layer, window query) when
  // summing, one per KV head when each group contributes its maximum
  const int terms_per_query = p->aggregate == KV_AGG_MAX_GROUP ? c->n_kv_heads : p->n_q_heads;
  ea.mass_norm = 1.0 / ((double)c->n_layers * terms_per_query * p->window);
  ea.policy = p->policy;
  ea.item_shift = item_shift;
  ea.dt_steps = p->dt_steps;
  ea.region = p->region;
  ea.base_prio = p->base_prio;
  ea.decay_rate = p->decay_rate;
  ea.n_regions = p->n_regions;
  ea.rho = p->rho;
  ea.alpha = p->alpha;
  ea.tau = p->tau;
  ea.ewma = p->ewma;
  ea.clock = p->clock;
  ea.accum = p->accum;
  ea.span_id = p->span_id;
  ea.span_bonus = p->span_bonus;
  ea.n_spans = p->n_spans;
  ea.pinned_regions = p->pinned_regions;
  ea.n_sink = p->n_sink;
  ea.n_recent = p->n_recent;
  ea.token_pinned = p->token_pinned;
  ea.mass = p->mass;
  ea.token_score = p->token_score;
  ea.item_score = p->item_score;
  ea.item_pinned = p->item_pinned;
  ea.status = p->status;
  if ((e = launch_epilogue(ea, stream)) != hipSuccess) return hip_fail(e);
  if ((e = mark(4)) != hipSuccess) return hip_fail(e);
  return KV_OK;
}

int32_t kv_select_workspace_size(int64_t n_items, size_t* bytes) {
  if (!bytes || n_items <= 0) return KV_EINVAL;
  *bytes = select_workspace_bytes(n_items);
  return KV_OK;
}

int32_t kv_select(const float* item_score, const uint8_t* item_pinned, int64_t n_items,
                  int32_t item_tokens, int64_t n_tokens, int64_t budget_items, int32_t* keep_tokens,
                  int64_t keep_capacity, int64_t* n_keep, uint32_t* status, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (!item_score || !keep_tokens || !n_keep || n_items <= 0 || item_tokens <= 0) return KV_EINVAL;
  if (n_tokens <= 0 || n_tokens > 0x7FFFFFFFLL || budget_items < 0 || keep_capacity < 0)
    return KV_EINVAL;
  if ((n_tokens + item_tokens - 1) / item_tokens != n_items) return KV_EINVAL;
  if (!ws || ws_bytes < select_workspace_bytes(n_items)) return KV_EWORKSPACE;
  int32_t rc = check_device();
  if (rc) return rc;
  SelectArgs a;
  memset(&a, 0, sizeof(a));
  a.score = item_score;
  a.pinned = item_pinned;
  a.n_items = n_items;
  a.item_tokens = item_tokens;
  a.n_tokens = n_tokens;
  a.budget = budget_items;
  a.keep = keep_tokens;
  a.keep_capacity = keep_capacity;
  a.n_keep = n_keep;
  a.status = status;
  a.n_blocks = select_blocks(n_items);
  a.per_block = (n_items + a.n_blocks - 1) / a.n_blocks;
  char* w = (char*)ws;
  a.st = (SelectState*)w;
  a.hist = (uint32_t*)(w + 256);
  a.counts = (int64_t*)(w + 256 + (size_t)3 * kSelBins * sizeof(uint32_t));
  const hipError_t e = launch_select(a, stream);
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

int32_t kv_select_noalloc(const float* item_score, const uint8_t* item_pinned, int64_t n_items,
                          int32_t item_tokens, int64_t n_tokens, int64_t budget_items,
                          int32_t* keep_tokens, int64_t keep_capacity, int64_t* n_keep,
                          uint32_t* status, hipStream_t stream) {
  if (n_items > 0 && select_workspace_bytes(n_items) > kSelectScratchBytes) return KV_EWORKSPACE;
  int32_t rc = check_device();
  if (rc) return rc;
  void* ws = nullptr;
  const hipError_t e = select_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e);
  return kv_select(item_score, item_pinned, n_items, item_tokens, n_tokens, budget_items, keep_tokens,
                   keep_capacity, n_keep, status, ws, kSelectScratchBytes, stream);
}

int32_t kv_lrfu_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes || n <= 0) return KV_EINVAL;
  *bytes = lrfu_workspace_bytes(n);
  return KV_OK;
}

int32_t kv_lrfu_update(const float* attn_score, int64_t n, float scale, float top_p, float decay,
                       float* keep_score, uint8_t* hit, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!attn_score || !keep_score || n <= 0 || n > 0x7FFFFFFFLL) return KV_EINVAL;
  if (!(top_p >= 0.f && top_p <= 1.f) || !(decay >= 0.f && decay <= 1.f) || !isfinite(scale))
    return KV_EINVAL;
  if (!ws || ws_bytes < lrfu_workspace_bytes(n)) return KV_EWORKSPACE;
  int32_t rc = check_device();
  if (rc) return rc;
  LrfuArgs a;
  memset(&a, 0, sizeof(a));
  a.score = attn_score;
  a.scale = scale;
  a.n = n;
  a.top_p = top_p;
  a.decay = decay;
  a.keep_score = keep_score;
  a.hit = hit;
  a.n_blocks = lrfu_blocks(n);
  a.per_block = (n + a.n_blocks - 1) / a.n_blocks;
  char* w = (char*)ws;
  a.st = (ToppState*)w;
  a.hist = (unsigned long long*)(w + 256);
  a.counts = (int64_t*)(w + 256 + (size_t)3 * 2048 * sizeof(unsigned long long));
  const hipError_t e = launch_lrfu(a, stream);
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

int32_t kv_select_segment(int64_t n_tokens, int64_t prefix_len, int64_t evict_tokens, int32_t block,
                          int32_t* keep_tokens, int64_t keep_capacity, int64_t* n_keep_dev,
                          int64_t* n_keep_host, int64_t* evict_len_host, hipStream_t stream) {
  if (n_tokens <= 0 || n_tokens > 0x7FFFFFFFLL || prefix_len < 0 || prefix_len > n_tokens ||
      evict_tokens < 0 || block <= 0)
    return KV_EINVAL;
  int64_t e = (evict_tokens + block - 1) / block * block;
  if (e > n_tokens - prefix_len) e = n_tokens - prefix_len;
  const int64_t n_keep = n_tokens - e;
  if (n_keep_host) *n_keep_host = n_keep;
  if (evict_len_host) *evict_len_host = e;
  if (!keep_tokens && !n_keep_dev) return KV_OK;
  if (keep_tokens && keep_capacity < n_keep) return KV_EINVAL;
  int32_t rc = check_device();
  if (rc) return rc;
  const hipError_t he = launch_segment_keep(n_tokens, prefix_len, e, keep_tokens, keep_capacity,
                                            n_keep_dev, n_keep, stream);
  return he == hipSuccess ? KV_OK : hip_fail(he);
}

int32_t kv_rope_inv_freq(const kv_rope* rope, double* inv_freq) {
  if (!rope || !inv_freq) return KV_EINVAL;
  const int half = kHeadDim / 2;
  if (rope->kind == KV_ROPE_TABLE) {
    if (!rope->inv_freq) return KV_EINVAL;
    for (int i = 0; i < half; ++i) {
      if (!isfinite(rope->inv_freq[i])) return KV_EINVAL;
      inv_freq[i] = rope->inv_freq[i];
    }
    return KV_OK;
  }
  if (!(rope->base > 1.0) || !isfinite(rope->base)) return KV_EINVAL;
  const bool scaled = rope->kind != KV_ROPE_DEFAULT;
  if (scaled && !(rope->factor > 0.0 && isfinite(rope->factor))) return KV_EINVAL;
  const double L = (double)rope->original_max_position;
  if ((rope->kind == KV_ROPE_LLAMA3 || rope->kind == KV_ROPE_YARN || rope->kind == KV_ROPE_YARN_RATIO) &&
      !(L > 0.0))
    return KV_EINVAL;
  if (rope->kind == KV_ROPE_LLAMA3 &&
      !(rope->low_freq_factor > 0.0 && rope->high_freq_factor > rope->low_freq_factor))
    return KV_EINVAL;
  const bool yarn = rope->kind == KV_ROPE_YARN || rope->kind == KV_ROPE_YARN_RATIO;
  if (yarn && !(rope->beta_fast > rope->beta_slow && rope->beta_slow > 0.0)) return KV_EINVAL;
  if (rope->kind < KV_ROPE_DEFAULT || rope->kind > KV_ROPE_YARN_RATIO || rope->kind == KV_ROPE_TABLE)
    return KV_EINVAL;
  if (rope->flags & ~(int32_t)KV_ROPE_YARN_NO_TRUNCATE) return KV_EINVAL;
  const double two_pi = 6.283185307179586476925286766559;
  // YaRN's blend band in pair indices: pair i turns L * f_i / (2 pi) times over the
  // original context, so it turns beta times at i(beta) = D ln(L / (2 pi beta)) / (2 ln base)
  double lo = 0.0, hi = 1.0;
  if (rope->kind == KV_ROPE_YARN) {
    lo = kHeadDim * log(L / (two_pi * rope->beta_fast)) / (2.0 * log(rope->base));
    hi = kHeadDim * log(L / (two_pi * rope->beta_slow)) / (2.0 * log(rope->base));
    if (!(rope->flags & KV_ROPE_YARN_NO_TRUNCATE)) {
      lo = floor(lo);
      hi = ceil(hi);
    }
    if (lo < 0.0) lo = 0.0;
    if (hi > kHeadDim - 1) hi = kHeadDim - 1;
    if (hi == lo) hi += 0.001;
  }
  for (int i = 0; i < half; ++i) {
    const double f = pow(rope->base, -(2.0 * i) / kHeadDim);
    double out = f;
    if (rope->kind == KV_ROPE_LINEAR) {
      out = f / rope->factor;
    } else if (rope->kind == KV_ROPE_LLAMA3) {
      const double w = two_pi / f;
      if (w < L / rope->high_freq_factor) {
        out = f;
      } else if (w > L / rope->low_freq_factor) {
        out = f / rope->factor;
      } else {
        const double t = (L / w - rope->low_freq_factor) / (rope->high_freq_factor - rope->low_freq_factor);
        out = (1.0 - t) * f / rope->factor + t * f;
      }
    } else if (rope->kind == KV_ROPE_YARN) {
      double g = (i - lo) / (hi - lo);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      out = g * f / rope->factor + (1.0 - g) * f;
    } else if (rope->kind == KV_ROPE_YARN_RATIO) {
      const double rot = L / (two_pi / f);
      double g = (rot - rope->beta_slow) / (rope->beta_fast - rope->beta_slow);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      out = (1.0 - g) * f / rope->factor + g * f;
    }
    inv_freq[i] = out;
  }
  return KV_OK;
}

// [a, a + an) and [b, b + bn) share a byte
static bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn) {
  const uint64_t x = (uint64_t)(uintptr_t)a, y = (uint64_t)(uintptr_t)b;
  return an && bn && x < y + bn && y < x + an;
}

// Bytes a cache without a block table spans from its base pointer (the last layer's
// pages of its n_tokens); 0 when a block table places pages anywhere.
static uint64_t cache_extent(const kv_cache_desc* c) {
  if (c->block_table) return 0;
  const int64_t pages = (c->n_tokens + c->page_size - 1) / c->page_size;
  return ((uint64_t)(c->n_layers - 1) * (uint64_t)c->layer_stride + (uint64_t)pages * (uint64_t)c->page_stride) * 2u;
}

// The gather form reads and writes different memory (ActKV Sec. 7.2 names the hazard of
// overlapping an in-place copy): its K/V extents (known without block tables), its
// positions and its metadata arrays must not overlap.
static int32_t check_disjoint(const kv_cache_desc* src, const kv_cache_desc* dst, const int32_t* old_pos,
                              const int32_t* new_pos, int64_t max_keep, const MetaSet& ms) {
  const uint64_t se = cache_extent(src), de = cache_extent(dst);
  const void* sp[2] = {src->k, src->v};
  const void* dp[2] = {dst->k, dst->v};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      if (overlaps(sp[i], se, dp[j], de)) return KV_EINVAL;
  if (new_pos && overlaps(old_pos, (uint64_t)src->n_tokens * 4u, new_pos, (uint64_t)max_keep * 4u)) return KV_EINVAL;
  for (int m = 0; m < ms.n; ++m) {
    const uint64_t b = (uint64_t)ms.elem_bytes[m];
    if (overlaps(ms.src[m], (uint64_t)src->n_tokens * b, ms.dst[m], (uint64_t)max_keep * b)) return KV_EINVAL;
    if (new_pos && overlaps(ms.dst[m], (uint64_t)max_keep * b, new_pos, (uint64_t)max_keep * 4u)) return KV_EINVAL;
  }
  return KV_OK;
}

static int32_t check_ref(const kv_ref_store* r, const kv_cache_desc* c, int64_t min_slots) {
  if (!r->k || !r->pos || r->n_slots < min_slots || r->n_slots <= 0) return KV_EINVAL;
  const int64_t slot = (int64_t)c->n_kv_heads * kHeadDim;
  if (c->n_layers > 1 && r->layer_stride < r->n_slots * slot) return KV_EINVAL;
  if (((uintptr_t)r->k & 15) || (r->layer_stride & 7)) return KV_EINVAL;
  return KV_OK;
}

static void fill_compact_common(CompactArgs* a, const kv_cache_desc* src, const kv_cache_desc* dst,
                                int32_t renumber_base, const double* inv_freq) {
  a->src_k = (const uint16_t*)src->k;
  a->src_v = (const uint16_t*)src->v;
  a->src_layer_stride = src->layer_stride;
  a->src_page_stride = src->page_stride;
  a->src_bt = src->block_table;
  a->dst_k = (uint16_t*)dst->k;
  a->dst_v = (uint16_t*)dst->v;
  a->dst_layer_stride = dst->layer_stride;
  a->dst_page_stride = dst->page_stride;
  a->dst_bt = dst->block_table;
  a->n_layers = src->n_layers;
  a->n_kv_heads = src->n_kv_heads;
  a->src_tokens = src->n_tokens;
  a->src_page_shift = log2_exact(src->page_size);
  a->dst_page_shift = log2_exact(dst->page_size);
  a->renumber_base = renumber_base;
  a->parts = 1;
  for (int i = 0; i < kHeadDim / 2; ++i) a->inv_freq[i] = inv_freq[i];
}

// Without a reference store a rank's copy is split over several workgroups (its
// positions and metadata are read and written by the first one only).  The store's check
// covers the whole key, so that path keeps one workgroup per rank.
static void fill_ref(CompactArgs* a, const kv_ref_store* src, const kv_ref_store* dst) {
  if (!src) {
    a->parts = compact_parts(a->n_layers, a->n_kv_heads);
    return;
  }
  a->ref_src_k = (const uint16_t*)src->k;
  a->ref_src_pos = src->pos;
  a->ref_src_layer_stride = src->layer_stride;
  a->ref_dst_k = (uint16_t*)dst->k;
  a->ref_dst_pos = dst->pos;
  a->ref_dst_layer_stride = dst->layer_stride;
}

static int32_t rope_table(const kv_rope* rope, double* inv_freq) {
  kv_rope def;
  memset(&def, 0, sizeof(def));
  def.kind = KV_ROPE_DEFAULT;
  def.base = 1e6;
  return kv_rope_inv_freq(rope ? rope : &def, inv_freq);
}

int32_t kv_ref_invalidate(const kv_ref_store* ref, int64_t first, int64_t count, hipStream_t stream) {
  if (!ref || !ref->pos || first < 0 || count < 0 || first + count > ref->n_slots) return KV_EINVAL;
  if (count == 0) return KV_OK;
  int32_t rc = check_device();
  if (rc) return rc;
  const hipError_t e = launch_ref_invalidate(ref->pos + first, count, stream);
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

int32_t kv_compact_rerope_ex(const kv_cache_desc* src, const kv_cache_desc* dst,
                             const int32_t* keep_tokens, const int64_t* n_keep, int64_t max_keep,
                             const int32_t* old_pos, int32_t* new_pos, int32_t renumber_base,
                             const kv_rope* rope, int32_t limit, const kv_meta_desc* meta,
                             int32_t n_meta, const kv_ref_store* ref_src, const kv_ref_store* ref_dst,
                             hipStream_t stream) {
  int32_t rc = check_cache(src);
  if (rc) return rc;
  if ((rc = check_cache(dst))) return rc;
  if (!keep_tokens || !old_pos || max_keep < 0) return KV_EINVAL;
  if (dst->n_layers != src->n_layers || dst->n_kv_heads != src->n_kv_heads) return KV_EINVAL;
  if (max_keep > dst->n_tokens || max_keep > src->n_tokens) return KV_EINVAL;
  if (src->k == dst->k || src->v == dst->v) return KV_EINVAL;
  double inv_freq[kHeadDim / 2];
  if ((rc = rope_table(rope, inv_freq))) return rc;
  if ((ref_src == nullptr) != (ref_dst == nullptr)) return KV_EINVAL;
  if (ref_src) {
    if ((rc = check_ref(ref_src, src, src->n_tokens)) || (rc = check_ref(ref_dst, src, max_keep))) return rc;
    if (ref_src->k == ref_dst->k || ref_src->pos == ref_dst->pos) return KV_EINVAL;
  }
  if (renumber_base >= 0 && limit > 0 && (int64_t)renumber_base + max_keep > limit) return KV_ELIMIT;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  if ((rc = check_disjoint(src, dst, old_pos, new_pos, max_keep, ms))) return rc;
  if (max_keep == 0) return KV_OK;
  if ((rc = check_device())) return rc;
  CompactArgs a;
  memset(&a, 0, sizeof(a));
  fill_compact_common(&a, src, dst, renumber_base, inv_freq);
  fill_ref(&a, ref_src, ref_dst);
  a.keep = keep_tokens;
  a.rank0 = 0;
  a.rank1 = max_keep;
  a.n_keep = n_keep;
  a.old_pos = old_pos;
  a.new_pos = new_pos;
  a.meta = ms;
  hipError_t e = launch_compact(a, stream);
  if (e != hipSuccess) return hip_fail(e);
  return KV_OK;
}

int32_t kv_compact_rerope(const kv_cache_desc* src, const kv_cache_desc* dst,
                          const int32_t* keep_tokens, const int64_t* n_keep, int64_t max_keep,
                          const int32_t* old_pos, int32_t* new_pos, int32_t renumber_base,
                          double rope_theta, int32_t limit, const kv_meta_desc* meta,
                          int32_t n_meta, hipStream_t stream) {
  kv_rope rope;
  memset(&rope, 0, sizeof(rope));
  rope.kind = KV_ROPE_DEFAULT;
  rope.base = rope_theta;
  return kv_compact_rerope_ex(src, dst, keep_tokens, n_keep, max_keep, old_pos, new_pos, renumber_base,
                              &rope, limit, meta, n_meta, nullptr, nullptr, stream);
}

int32_t kv_compact_segment_inplace_ex(const kv_cache_desc* cache, int64_t prefix_len, int64_t evict_len,
                                      int32_t* pos, int32_t renumber_base, const kv_rope* rope,
                                      int32_t limit, const kv_meta_desc* meta, int32_t n_meta,
                                      const kv_ref_store* ref, hipStream_t stream) {
  int32_t rc = check_cache(cache);
  if (rc) return rc;
  const int64_t N = cache->n_tokens;
  if (!pos || prefix_len < 0 || evict_len < 0 || prefix_len + evict_len > N) return KV_EINVAL;
  double inv_freq[kHeadDim / 2];
  if ((rc = rope_table(rope, inv_freq))) return rc;
  if (ref && (rc = check_ref(ref, cache, N))) return rc;
  const int64_t n_keep = N - evict_len;
  if (renumber_base >= 0 && limit > 0 && (int64_t)renumber_base + n_keep > limit) return KV_ELIMIT;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  for (int i = 0; i < ms.n; ++i)
    if (ms.src[i] != ms.dst[i]) return KV_EINVAL;
  if ((rc = check_device())) return rc;
  CompactArgs a;
  memset(&a, 0, sizeof(a));
  fill_compact_common(&a, cache, cache, renumber_base, inv_freq);
  fill_ref(&a, ref, ref);
  a.keep = nullptr;
  a.split = prefix_len;
  a.shift = evict_len;
  a.n_keep = nullptr;
  a.old_pos = pos;
  a.new_pos = pos;
  a.meta = ms;
  a.rows_in_place = 1;
  hipError_t e;
  // prefix: stays in place (re-rotated only if its positions change); a rank reads and
  // writes its own position here, so each rank is one workgroup
  const int parts = a.parts;
  a.rank0 = 0;
  a.rank1 = prefix_len;
  a.parts = 1;
  if ((e = launch_compact(a, stream)) != hipSuccess) return hip_fail(e);
  a.parts = parts;
  if (evict_len == 0) return KV_OK;
  // suffix: rounds of at most evict_len ranks; round k reads [r0+E, r1+E) and writes
  // [r0, r1), disjoint because r1 - r0 <= E; later rounds read only beyond r1 + E.
  for (int64_t r0 = prefix_len; r0 < n_keep; r0 += evict_len) {
    a.rank0 = r0;
    a.rank1 = r0 + evict_len < n_keep ? r0 + evict_len : n_keep;
    if ((e = launch_compact(a, stream)) != hipSuccess) return hip_fail(e);
  }
  return KV_OK;
}

int32_t kv_gather_evicted(const kv_cache_desc* src, const int32_t* keep_tokens, int64_t n_keep,
                          int64_t first, int64_t count, const kv_cache_desc* dst, int32_t* evicted_tokens,
                          const kv_meta_desc* meta, int32_t n_meta, hipStream_t stream) {
  int32_t rc = check_cache(src);
  if (rc) return rc;
  if ((rc = check_cache(dst))) return rc;
  if ((n_keep > 0 && !keep_tokens) || n_keep < 0 || n_keep > src->n_tokens) return KV_EINVAL;
  if (first < 0 || count < 0 || first + count > src->n_tokens - n_keep || dst->n_tokens < count) return KV_EINVAL;
  if (dst->n_layers != src->n_layers || dst->n_kv_heads != src->n_kv_heads) return KV_EINVAL;
  if (src->k == dst->k || src->v == dst->v) return KV_EINVAL;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  if (count == 0) return KV_OK;
  if ((rc = check_device())) return rc;
  EvictArgs a;
  memset(&a, 0, sizeof(a));
  a.src_k = (const uint16_t*)src->k;
  a.src_v = (const uint16_t*)src->v;
  a.src_layer_stride = src->layer_stride;
  a.src_page_stride = src->page_stride;
  a.src_bt = src->block_table;
  a.src_page_shift = log2_exact(src->page_size);
  a.dst_k = (uint16_t*)dst->k;
  a.dst_v = (uint16_t*)dst->v;
  a.dst_layer_stride = dst->layer_stride;
  a.dst_page_stride = dst->page_stride;
  a.dst_bt = dst->block_table;
  a.dst_page_shift = log2_exact(dst->page_size);
  a.n_layers = src->n_layers;
  a.n_kv_heads = src->n_kv_heads;
  a.keep = keep_tokens;
  a.n_keep = n_keep;
  a.src_tokens = src->n_tokens;
  a.first = first;
  a.count = count;
  a.evicted_tokens = evicted_tokens;
  a.meta = ms;
  const hipError_t e = launch_gather_evicted(a, stream);
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

static size_t offload_row_bytes(const kv_cache_desc* src, int64_t chunk) {
  return align256((size_t)chunk * src->n_layers * src->n_kv_heads * kHeadDim * sizeof(uint16_t));
}

int32_t kv_offload_workspace_size(const kv_cache_desc* src, int64_t chunk, size_t* bytes) {
  int32_t rc = check_cache(src);
  if (rc) return rc;
  if (!bytes || chunk <= 0) return KV_EINVAL;
  *bytes = 2 * offload_row_bytes(src, chunk) + align256((size_t)chunk * sizeof(int32_t));
  return KV_OK;
}

int32_t kv_offload_evicted(const kv_cache_desc* src, const int32_t* keep_tokens, int64_t n_keep, int64_t chunk,
                           void* host_k, void* host_v, int32_t* host_tokens, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  size_t need = 0;
  int32_t rc = kv_offload_workspace_size(src, chunk, &need);
  if (rc) return rc;
  if (!host_k || !host_v || n_keep < 0 || n_keep > src->n_tokens || (n_keep > 0 && !keep_tokens)) return KV_EINVAL;
  if (!ws || ws_bytes < need) return KV_EWORKSPACE;
  const int64_t n_ev = src->n_tokens - n_keep;
  if (n_ev == 0) return KV_OK;
  if ((rc = check_device())) return rc;
  const int64_t slot = (int64_t)src->n_kv_heads * kHeadDim;
  char* w = (char*)ws;
  kv_cache_desc stage;
  memset(&stage, 0, sizeof(stage));
  stage.k = w;
  stage.v = w + offload_row_bytes(src, chunk);
  stage.n_layers = src->n_layers;
  stage.n_kv_heads = src->n_kv_heads;
  stage.head_dim = kHeadDim;
  stage.page_size = 1;
  stage.n_tokens = chunk;
  stage.page_stride = slot;
  stage.layer_stride = chunk * slot;
  stage.block_table = nullptr;
  int32_t* ids = (int32_t*)(w + 2 * offload_row_bytes(src, chunk));
  const size_t row_bytes = (size_t)slot * sizeof(uint16_t);
  for (int64_t e0 = 0; e0 < n_ev; e0 += chunk) {
    const int64_t cnt = n_ev - e0 < chunk ? n_ev - e0 : chunk;
    if ((rc = kv_gather_evicted(src, keep_tokens, n_keep, e0, cnt, &stage, ids, nullptr, 0, stream))) return rc;
    hipError_t e;
    for (int which = 0; which < 2; ++which) {
      char* host = (char*)(which ? host_v : host_k) + (size_t)e0 * row_bytes;
      const char* dev = (const char*)(which ? stage.v : stage.k);
      e = hipMemcpy2DAsync(host, (size_t)n_ev * row_bytes, dev, (size_t)chunk * row_bytes,
                           (size_t)cnt * row_bytes, (size_t)src->n_layers, hipMemcpyDeviceToHost, stream);
      if (e != hipSuccess) return hip_fail(e);
    }
    if (host_tokens) {
      e = hipMemcpyAsync(host_tokens + e0, ids, (size_t)cnt * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  return KV_OK;
}

// Staging rows of the offload / load / swap workspace: chunk tokens of K, then of V,
// layer-major, then chunk int32 ids.
static kv_cache_desc staging_desc(const kv_cache_desc* like, void* ws, int64_t chunk) {
  kv_cache_desc st;
  memset(&st, 0, sizeof(st));
  const int64_t slot = (int64_t)like->n_kv_heads * kHeadDim;
  st.k = ws;
  st.v = (char*)ws + offload_row_bytes(like, chunk);
  st.n_layers = like->n_layers;
  st.n_kv_heads = like->n_kv_heads;
  st.head_dim = kHeadDim;
  st.page_size = 1;
  st.n_tokens = chunk;
  st.page_stride = slot;
  st.layer_stride = chunk * slot;
  st.block_table = nullptr;
  return st;
}

static MoveArgs move_args(const kv_cache_desc* src, const kv_cache_desc* dst) {
  MoveArgs a;
  memset(&a, 0, sizeof(a));
  a.src_k = (const uint16_t*)src->k;
  a.src_v = (const uint16_t*)src->v;
  a.src_layer_stride = src->layer_stride;
  a.src_page_stride = src->page_stride;
  a.src_bt = src->block_table;
  a.src_page_shift = log2_exact(src->page_size);
  a.src_tokens = src->n_tokens;
  a.dst_k = (uint16_t*)dst->k;
  a.dst_v = (uint16_t*)dst->v;
  a.dst_layer_stride = dst->layer_stride;
  a.dst_page_stride = dst->page_stride;
  a.dst_bt = dst->block_table;
  a.dst_page_shift = log2_exact(dst->page_size);
  a.dst_tokens = dst->n_tokens;
  a.n_layers = src->n_layers;
  a.n_kv_heads = src->n_kv_heads;
  return a;
}

// One chunk's K and V between host rows [host_row, host_row + cnt) of a [L][host_rows]
// pool and the staging rows, every layer (one 2D copy per array).
static hipError_t host_chunk_copy(const kv_cache_desc* c, const kv_cache_desc* stage, void* host_k,
                                  void* host_v, int64_t host_rows, int64_t host_row, int64_t cnt,
                                  int64_t chunk, bool to_host, hipStream_t stream) {
  const size_t row_bytes = (size_t)c->n_kv_heads * kHeadDim * sizeof(uint16_t);
  for (int which = 0; which < 2; ++which) {
    char* host = (char*)(which ? host_v : host_k) + (size_t)host_row * row_bytes;
    char* dev = (char*)(which ? stage->v : stage->k);
    const hipError_t e =
        to_host ? hipMemcpy2DAsync(host, (size_t)host_rows * row_bytes, dev, (size_t)chunk * row_bytes,
                                   (size_t)cnt * row_bytes, (size_t)c->n_layers, hipMemcpyDeviceToHost, stream)
                : hipMemcpy2DAsync(dev, (size_t)chunk * row_bytes, host, (size_t)host_rows * row_bytes,
                                   (size_t)cnt * row_bytes, (size_t)c->n_layers, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int32_t kv_load_rows(const kv_cache_desc* dst, const int32_t* slots, int64_t count, const void* host_k,
                     const void* host_v, int64_t host_rows, int64_t host_first, int64_t chunk,
                     const kv_meta_desc* meta, int32_t n_meta, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  size_t need = 0;
  int32_t rc = kv_offload_workspace_size(dst, chunk, &need);
  if (rc) return rc;
  if (count < 0 || (count > 0 && (!slots || !host_k || !host_v))) return KV_EINVAL;
  if (host_first < 0 || host_rows < 0 || host_first + count > host_rows) return KV_EINVAL;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  if (!ws || ws_bytes < need) return KV_EWORKSPACE;
  if (count == 0) return KV_OK;
  if ((rc = check_device())) return rc;
  const kv_cache_desc stage = staging_desc(dst, ws, chunk);
  MoveArgs a = move_args(&stage, dst);
  a.meta = ms;
  for (int64_t c0 = 0; c0 < count; c0 += chunk) {
    const int64_t cnt = count - c0 < chunk ? count - c0 : chunk;
    hipError_t e = host_chunk_copy(dst, &stage, (void*)host_k, (void*)host_v, host_rows, host_first + c0, cnt,
                                   chunk, false, stream);
    if (e != hipSuccess) return hip_fail(e);
    a.src_rows = nullptr;
    a.src_first = 0;
    a.dst_rows = slots + c0;
    a.meta_first = c0;
    a.count = cnt;
    if ((e = launch_move_rows(a, stream)) != hipSuccess) return hip_fail(e);
  }
  return KV_OK;
}

int32_t kv_swap_workspace_size(const kv_cache_desc* cache, int64_t chunk, size_t* bytes) {
  size_t one = 0;
  const int32_t rc = kv_offload_workspace_size(cache, chunk, &one);
  if (rc) return rc;
  *bytes = 2 * one;   // one staging area per direction
  return KV_OK;
}

int32_t kv_swap_chunked(const kv_cache_desc* cache, const int32_t* slots, int64_t count, void* host_k,
                        void* host_v, int64_t host_rows, int64_t in_first, int64_t buf_first, int64_t chunk,
                        int64_t* out_rows, int64_t* next_buf_first, void* ws, size_t ws_bytes,
                        hipStream_t stream, hipStream_t in_stream) {
  size_t need = 0;
  int32_t rc = kv_swap_workspace_size(cache, chunk, &need);
  if (rc) return rc;
  if (count < 0 || (count > 0 && (!slots || !host_k || !host_v))) return KV_EINVAL;
  if (in_first < 0 || buf_first < 0 || in_first + count > host_rows) return KV_EINVAL;
  const int64_t first_n = count < chunk ? count : chunk;
  if (buf_first + first_n > host_rows) return KV_EINVAL;
  if (count > 0 && buf_first < in_first + count && in_first < buf_first + first_n) return KV_EINVAL;
  if (!ws || ws_bytes < need) return KV_EWORKSPACE;
  // where every outgoing row lands: the buffer, then the rows each incoming chunk frees
  int64_t buf = buf_first;
  for (int64_t c0 = 0; c0 < count; c0 += chunk) {
    const int64_t cnt = count - c0 < chunk ? count - c0 : chunk;
    if (out_rows)
      for (int64_t r = 0; r < cnt; ++r) out_rows[c0 + r] = buf + r;
    buf = in_first + c0;
  }
  if (next_buf_first) *next_buf_first = buf;
  if (count == 0) return KV_OK;
  if ((rc = check_device())) return rc;
  // Outgoing chunks (gather, device-to-host) run on `stream` through the first staging
  // area, incoming ones (host-to-device, scatter) on `in_stream` through the second, so
  // that the two directions of the link overlap.  Two orderings cross the streams: chunk
  // c's scatter overwrites the slots its gather reads, and chunk c's device-to-host copy
  // overwrites the CPU rows chunk c-1's host-to-device copy reads (its buffer).
  const bool two = in_stream != stream;
  size_t one = 0;
  kv_offload_workspace_size(cache, chunk, &one);
  const kv_cache_desc st_out = staging_desc(cache, ws, chunk);
  const kv_cache_desc st_in = staging_desc(cache, (char*)ws + one, chunk);
  MoveArgs out = move_args(cache, &st_out);
  MoveArgs in = move_args(&st_in, cache);
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};   // start, gathered, read from the host
  hipError_t e = hipSuccess;
  auto cleanup = [&]() {
    for (hipEvent_t x : ev)
      if (x) (void)hipEventDestroy(x);   // released once the work recorded on it has completed
  };
  if (two) {
    for (hipEvent_t& x : ev)
      if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
        cleanup();
        return hip_fail(e);
      }
    // the incoming side starts after the work enqueued so far on `stream`
    if ((e = hipEventRecord(ev[0], stream)) != hipSuccess || (e = hipStreamWaitEvent(in_stream, ev[0], 0)) != hipSuccess) {
      cleanup();
      return hip_fail(e);
    }
  }
  hipStream_t sin = two ? in_stream : stream;
  buf = buf_first;
  for (int64_t c0 = 0; c0 < count && e == hipSuccess; c0 += chunk) {
    const int64_t cnt = count - c0 < chunk ? count - c0 : chunk;
    // the chunk leaving the GPU: gathered, then written into the current CPU buffer once
    // the previous incoming chunk has been read from those rows
    out.src_rows = slots + c0;
    out.dst_rows = nullptr;
    out.dst_first = 0;
    out.count = cnt;
    if ((e = launch_move_rows(out, stream)) != hipSuccess) break;
    if (two && (e = hipEventRecord(ev[1], stream)) != hipSuccess) break;
    if (two && c0 > 0 && (e = hipStreamWaitEvent(stream, ev[2], 0)) != hipSuccess) break;
    if ((e = host_chunk_copy(cache, &st_out, host_k, host_v, host_rows, buf, cnt, chunk, true, stream)) != hipSuccess)
      break;
    // the chunk coming from the CPU: into the GPU slots freed once they are gathered
    if ((e = host_chunk_copy(cache, &st_in, host_k, host_v, host_rows, in_first + c0, cnt, chunk, false, sin)) !=
        hipSuccess)
      break;
    if (two && (e = hipEventRecord(ev[2], sin)) != hipSuccess) break;
    if (two && (e = hipStreamWaitEvent(sin, ev[1], 0)) != hipSuccess) break;
    in.src_rows = nullptr;
    in.src_first = 0;
    in.dst_rows = slots + c0;
    in.count = cnt;
    if ((e = launch_move_rows(in, sin)) != hipSuccess) break;
    buf = in_first + c0;   // the CPU rows this chunk emptied are the next buffer
  }
  // the call completes on `stream`
  if (e == hipSuccess && two && (e = hipEventRecord(ev[2], sin)) == hipSuccess)
    e = hipStreamWaitEvent(stream, ev[2], 0);
  cleanup();
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

int32_t kv_compact_tail_inplace(const kv_cache_desc* cache, const int32_t* keep_tokens,
                                const int64_t* n_keep, int64_t max_keep, int64_t budget,
                                const kv_meta_desc* meta, int32_t n_meta, int64_t* start_host,
                                uint32_t* status, hipStream_t stream) {
  int32_t rc = check_cache(cache);
  if (rc) return rc;
  if (!keep_tokens || max_keep < 0 || max_keep > cache->n_tokens || budget <= 0) return KV_EINVAL;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  for (int i = 0; i < ms.n; ++i)
    if (ms.src[i] != ms.dst[i]) return KV_EINVAL;
  const int64_t N = cache->n_tokens, blk = cache->page_size;
  const int64_t y = (N + blk - 1) / blk, x = (budget + blk - 1) / blk;
  const int64_t start = budget >= N ? 0 : (y - x) * blk;
  if (start_host) *start_host = start;
  if ((rc = check_device())) return rc;
  TailArgs a;
  memset(&a, 0, sizeof(a));
  a.k = (uint16_t*)cache->k;
  a.v = (uint16_t*)cache->v;
  a.layer_stride = cache->layer_stride;
  a.page_stride = cache->page_stride;
  a.bt = cache->block_table;
  a.n_layers = cache->n_layers;
  a.n_kv_heads = cache->n_kv_heads;
  a.page_shift = log2_exact(cache->page_size);
  a.keep = keep_tokens;
  a.n_keep = n_keep;
  a.max_keep = max_keep;
  a.n_tokens = N;
  a.start = start;
  a.budget = budget >= N ? N : budget;
  a.status = status;
  a.meta = ms;
  const int64_t grid = max_keep < a.budget ? max_keep : a.budget;
  const hipError_t e = launch_tail_compact(a, grid, stream);
  return e == hipSuccess ? KV_OK : hip_fail(e);
}

int32_t kv_compact_segment_remap(const kv_cache_desc* cache, int64_t prefix_len, int64_t evict_len,
                                 int32_t* block_table_out, int32_t* freed_pages, const int32_t* old_pos,
                                 int32_t* new_pos, int32_t renumber_base, const kv_rope* rope, int32_t limit,
                                 const kv_meta_desc* meta, int32_t n_meta, hipStream_t stream) {
  int32_t rc = check_cache(cache);
  if (rc) return rc;
  const int64_t N = cache->n_tokens, pg = cache->page_size;
  if (!cache->block_table || !block_table_out || !old_pos || !new_pos) return KV_EINVAL;
  if (prefix_len < 0 || evict_len < 0 || prefix_len + evict_len > N) return KV_EINVAL;
  if (prefix_len % pg || evict_len % pg) return KV_EINVAL;   // whole pages only
  double inv_freq[kHeadDim / 2];
  if ((rc = rope_table(rope, inv_freq))) return rc;
  const int64_t n_keep = N - evict_len;
  if (renumber_base >= 0 && limit > 0 && (int64_t)renumber_base + n_keep > limit) return KV_ELIMIT;
  const int64_t n_pages = (N + pg - 1) / pg, keep_pages = (n_keep + pg - 1) / pg, evict_pages = evict_len / pg;
  // every output lands in memory that no input of the call occupies
  const uint64_t bt_bytes = (uint64_t)n_pages * 4u, out_bytes = (uint64_t)keep_pages * 4u;
  if (overlaps(cache->block_table, bt_bytes, block_table_out, out_bytes)) return KV_EINVAL;
  if (freed_pages && (overlaps(cache->block_table, bt_bytes, freed_pages, (uint64_t)evict_pages * 4u) ||
                      overlaps(block_table_out, out_bytes, freed_pages, (uint64_t)evict_pages * 4u)))
    return KV_EINVAL;
  if (overlaps(old_pos, (uint64_t)N * 4u, new_pos, (uint64_t)n_keep * 4u)) return KV_EINVAL;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  for (int m = 0; m < ms.n; ++m) {
    const uint64_t b = (uint64_t)ms.elem_bytes[m];
    if (overlaps(ms.src[m], (uint64_t)N * b, ms.dst[m], (uint64_t)n_keep * b) ||
        overlaps(ms.dst[m], (uint64_t)n_keep * b, new_pos, (uint64_t)n_keep * 4u))
      return KV_EINVAL;
  }
  if ((rc = check_device())) return rc;
  hipError_t e = launch_remap_table(cache->block_table, block_table_out, freed_pages, keep_pages,
                                    prefix_len / pg, evict_pages, stream);
  if (e != hipSuccess) return hip_fail(e);
  // every kept token keeps its physical slot: rank r's slot under the new table is its
  // source token's slot under the old one, so keys are re-rotated in place and values
  // stay where they are; no rank writes what another reads, so one launch covers all
  kv_cache_desc out = *cache;
  out.block_table = block_table_out;
  out.n_tokens = n_keep;
  CompactArgs a;
  memset(&a, 0, sizeof(a));
  fill_compact_common(&a, cache, &out, renumber_base, inv_freq);
  fill_ref(&a, nullptr, nullptr);
  a.keep = nullptr;
  a.split = prefix_len;
  a.shift = evict_len;
  a.n_keep = nullptr;
  a.old_pos = old_pos;
  a.new_pos = new_pos;
  a.meta = ms;
  a.rows_in_place = 0;
  a.remap_only = 1;
  a.rank0 = 0;
  a.rank1 = n_keep;
  // One workgroup per rank: with values untouched a rank's key is little work, and
  // splitting it (as the moving forms do) made the Mistral-7B row slower (measured: 8
  // workgroups per rank 2.32-2.38 ms, 4 2.11-2.12, 2 2.15, 1 2.04 ms).
  a.parts = 1;
  // without renumbering no position changes: positions and metadata only
  if (renumber_base < 0) e = launch_remap_rows(a, n_keep, stream);
  else e = launch_compact(a, stream);
  if (e != hipSuccess) return hip_fail(e);
  return KV_OK;
}

int32_t kv_compact_pages_remap(const kv_cache_desc* cache, const int32_t* keep_tokens, const int64_t* n_keep,
                               int64_t max_keep, int32_t* block_table_out, const int32_t* old_pos,
                               int32_t* new_pos, int32_t renumber_base, const kv_rope* rope, int32_t limit,
                               const kv_meta_desc* meta, int32_t n_meta, uint32_t* status, hipStream_t stream) {
  int32_t rc = check_cache(cache);
  if (rc) return rc;
  const int64_t N = cache->n_tokens, pg = cache->page_size;
  if (!cache->block_table || !keep_tokens || !block_table_out || !old_pos || !new_pos) return KV_EINVAL;
  if (max_keep < 0 || max_keep > N) return KV_EINVAL;
  double inv_freq[kHeadDim / 2];
  if ((rc = rope_table(rope, inv_freq))) return rc;
  if (renumber_base >= 0 && limit > 0 && (int64_t)renumber_base + max_keep > limit) return KV_ELIMIT;
  const int64_t n_pages = (N + pg - 1) / pg, out_pages = (max_keep + pg - 1) / pg;
  const uint64_t bt_bytes = (uint64_t)n_pages * 4u, out_bytes = (uint64_t)out_pages * 4u;
  if (overlaps(cache->block_table, bt_bytes, block_table_out, out_bytes)) return KV_EINVAL;
  if (overlaps(keep_tokens, (uint64_t)max_keep * 4u, block_table_out, out_bytes)) return KV_EINVAL;
  if (overlaps(old_pos, (uint64_t)N * 4u, new_pos, (uint64_t)max_keep * 4u)) return KV_EINVAL;
  MetaSet ms;
  if ((rc = check_meta(meta, n_meta, &ms))) return rc;
  for (int m = 0; m < ms.n; ++m) {
    const uint64_t b = (uint64_t)ms.elem_bytes[m];
    if (overlaps(ms.src[m], (uint64_t)N * b, ms.dst[m], (uint64_t)max_keep * b) ||
        overlaps(ms.dst[m], (uint64_t)max_keep * b, new_pos, (uint64_t)max_keep * 4u))
      return KV_EINVAL;
  }
  if ((rc = check_device())) return rc;
  hipError_t e = launch_remap_pages(cache->block_table, block_table_out, keep_tokens, n_keep, max_keep,
                                    log2_exact(pg), n_pages, status, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (max_keep == 0) return KV_OK;
  // every whole-page keep entry sits in the same physical slot under the new table, so
  // keys are re-rotated in place and values stay; one workgroup per rank, as for the
  // segment form
  kv_cache_desc out = *cache;
  out.block_table = block_table_out;
  out.n_tokens = max_keep;
  CompactArgs a;
  memset(&a, 0, sizeof(a));
  fill_compact_common(&a, cache, &out, renumber_base, inv_freq);
  fill_ref(&a, nullptr, nullptr);
  // One workgroup per rank (measured on a 1M-token page row with a 2,048-token budget:
  // 82.5 us, against 85-89 us with the gather's nine workgroups per rank, whose extra
  // workgroups mostly exit at once for ranks beyond the device count).
  a.parts = 1;
  a.keep = keep_tokens;
  a.n_keep = n_keep;
  a.old_pos = old_pos;
  a.new_pos = new_pos;
  a.meta = ms;
  a.remap_only = 1;
  a.status = status;
  a.rank0 = 0;
  a.rank1 = max_keep;
  if ((e = launch_compact(a, stream)) != hipSuccess) return hip_fail(e);
  return KV_OK;
}

int32_t kv_compact_segment_inplace(const kv_cache_desc* cache, int64_t prefix_len, int64_t evict_len,
                                   int32_t* pos, int32_t renumber_base, double rope_theta,
                                   int32_t limit, const kv_meta_desc* meta, int32_t n_meta,
                                   hipStream_t stream) {
  kv_rope rope;
  memset(&rope, 0, sizeof(rope));
  rope.kind = KV_ROPE_DEFAULT;
  rope.base = rope_theta;
  return kv_compact_segment_inplace_ex(cache, prefix_len, evict_len, pos, renumber_base, &rope, limit,
                                       meta, n_meta, nullptr, stream);
}

}  // extern "C"
