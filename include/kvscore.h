/*
 * kvscore.h -- C ABI of the MI355X (gfx950) KV-cache scoring / selection / compaction
 * library.
 *
 * The library implements, for one sequence row of a paged bf16 KV cache, the three
 * primitives that ActKV ("ActKV: Efficient LLM Agents through Action-Guided KV Cache
 * Management", Sec. 3.3) names for every score-based compression method,
 *     AttnScore <- CalAttn(q, K),  KeepMask <- Eviction(AttnScore, Budget),
 *     KV <- Compaction(KV, KeepMask),
 * plus PACE's bounded-position renumbering ("PACE: Keeping the Right Tokens in the KV
 * Cache Is Not Enough for Long-Horizon LLM Agents", Sec. 3.2, Proposition 1).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *   - The library never allocates device memory and keeps no mutable global state;
 *     scratch space is a caller-provided workspace sized by the *_workspace_size call.
 *     The one exception is kv_select_noalloc, which works in a fixed device array of its
 *     own for callers that cannot allocate (see there).
 *   - Work is enqueued asynchronously on the caller's stream; outputs are valid once the
 *     stream has reached that point.  Calls on different streams are independent as
 *     long as their buffers (workspaces included) do not overlap.
 *   - Errors are returned as int32 codes (KV_OK = 0, negative = error, positive =
 *     warning); nothing is enqueued when an error is returned for bad arguments.
 *     kv_strerror() describes a code.  Conditions that only the device can see (NaN
 *     scores, more pinned items than the budget) are reported in a device status word.
 */
#ifndef KVSCORE_H
#define KVSCORE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_ABI_VERSION 4

/* return codes */
#define KV_OK 0
#define KV_EINVAL (-1)        /* null pointer, bad size or stride, W > N, Hq % Hkv != 0 */
#define KV_EUNSUPPORTED (-2)  /* head_dim != 128, page size not a power of two <= 1024,
                                 more than 512 window rows per KV head (G*W, or
                                 pow2ceil(G)*W with KV_AGG_MAX_GROUP), G > 32 with
                                 KV_AGG_MAX_GROUP, or the device is not gfx950 */
#define KV_EWORKSPACE (-3)    /* workspace smaller than *_workspace_size reported */
#define KV_EHIP (-4)          /* a HIP call failed; kv_strerror appends its message */
#define KV_ELIMIT (-5)        /* renumbered row does not fit under the position limit */

/* bits of the device status word written by kv_select */
#define KV_STATUS_PINNED_OVER_BUDGET 1u /* pinned items alone exceed the budget: all of
                                           them are kept (MemDecay keeps pinned tokens
                                           unconditionally) and n_keep > budget */
#define KV_STATUS_NAN_SCORE 2u          /* some score was NaN; NaN orders after numbers */
#define KV_STATUS_KEEP_OVERFLOW 4u      /* keep list larger than keep_capacity; only the
                                           first keep_capacity entries were written */
/* bit of the device status word written by kv_score */
#define KV_STATUS_BAD_REGION 8u         /* some region label was >= n_regions */
/* bit of the device status word written by kv_compact_pages_remap */
#define KV_STATUS_NOT_WHOLE_PAGES 16u   /* some kept token would have to leave its slot (the
                                           keep list is not whole pages); it was not moved */

/*
 * One sequence row of a paged KV cache, all layers (ActKV Sec. 2.5: PagedKVCache
 * [2, B, BS, H, D] with a block table mapping logical token positions to blocks).
 * Element d of KV head h of logical token j in layer l lives at
 *     base + l*layer_stride + phys(j/page_size)*page_stride
 *          + (j%page_size)*n_kv_heads*head_dim + h*head_dim + d        (bf16 elements)
 * with phys(p) = block_table[p], or p when block_table is NULL.  k and v may share
 * one allocation (set v = k + offset).  All strides are in elements.
 */
typedef struct kv_cache_desc {
  void *k;                    /* bf16 keys (post-RoPE, as the model cached them) */
  void *v;                    /* bf16 values */
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t head_dim;           /* must be 128 */
  int32_t page_size;          /* power of two, 1..1024 */
  int64_t n_tokens;           /* N: logical tokens in the row */
  int64_t layer_stride;       /* elements between layers */
  int64_t page_stride;        /* elements between physical pages; >= page_size*Hkv*D,
                                 below 2^32 (else KV_EUNSUPPORTED) */
  const int32_t *block_table; /* device [ceil(N/page_size)] or NULL (identity) */
} kv_cache_desc;

/* Metadata array that travels with its token through compaction:
 * dst[r] = src[keep[r]] for element size elem_bytes (1, 2, 4 or 8). */
typedef struct kv_meta_desc {
  const void *src;
  void *dst;
  int32_t elem_bytes;
  int32_t reserved;
} kv_meta_desc;

#define KV_MAX_META 8

#define KV_POLICY_MEMDECAY 0 /* MemDecay region-decay score */
#define KV_POLICY_H2O 1      /* H2O accumulated attention (PACE's base policy) */

#define KV_AGG_SUM 0         /* sum the weights of every query head */
#define KV_AGG_MAX_GROUP 1   /* per KV head, the maximum over its GQA group (ActKV) */

/*
 * kv_score parameters.
 *
 * Attention mass (MemDecay, Method: the attention weight a token receives from the
 * window queries, taken as a mean over layers and heads; ActKV Sec. 2.3 / 7.1: A = exp(q.k - LSE); PACE Sec. 2: SnapKV window):
 * the W window queries are the last W tokens of the row.  For layer l, query head h
 * (KV head h / (Hq/Hkv)) and window query w at position N-W+w,
 *     s_j = scale * <q[l][w][h], k[l][j][h/G]>  for j <= N-W+w,
 *     LSE = log sum_j exp(s_j),  A_j = exp(s_j - LSE),
 *     KV_AGG_SUM:        mass_j = sum_{l,h,w} A_j;
 *     KV_AGG_MAX_GROUP:  mass_j = sum_{l,g,w} max_{h in group g} A_j   (ActKV Sec. 7.1,
 *                        Algorithm 3: the attention of a KV head is the maximum over
 *                        the query heads that share it).
 * When lse_in is given its values are used as LSE (no pass computes it).
 *
 * Policy epilogue, per token i:
 *   MEMDECAY (MemDecay, Method):  Abar = mass / T with T = L*Hq*W terms (KV_AGG_SUM)
 *       or T = L*Hkv*W (KV_AGG_MAX_GROUP);
 *       ewma <- rho*ewma + (1-rho)*Abar;  clock <- (Abar > tau) ? 0 : clock + dt_steps;
 *       s = base_prio[r]*exp(-decay_rate[r]*clock) + alpha*ewma + bonus
 *   H2O (PACE Sec. 2):  accum <- accum + mass;  s = accum + bonus
 * Foresight bonus (PACE Sec. 3.1 and 7): the planner turns its forward-reference table
 * into one bonus per span, soonest-needed spans highest and every needed span at or above
 * a constant floor; the library takes those values as input and adds
 * bonus = span_bonus[span_id[i]] to the token's score.  A span id outside [0, n_spans)
 * names no span (no bonus).
 * Pinned tokens (MemDecay pinned regions; PACE Table 1 sinks and recent window): a token
 * is pinned if its region bit is set in pinned_regions, or i < n_sink, or
 * i >= N - n_recent, or token_pinned[i] != 0.
 * A region label >= n_regions names no region: the token gets b = lambda = 0, no region
 * pinning, and KV_STATUS_BAD_REGION is set in *status.
 * Items: item_tokens == 1 scores tokens; item_tokens == page_size scores pages by the
 * mean of their tokens' scores (MemDecay S_p, over the tokens present) and pins a page
 * when any of its tokens is pinned.
 */
typedef struct kv_score_params {
  const void *q;              /* bf16 [L][W][Hq][128], rotated at their own positions */
  int32_t n_q_heads;          /* Hq, multiple of Hkv; G = Hq/Hkv (see KV_EUNSUPPORTED) */
  int32_t window;             /* W, 1..N */
  float scale;                /* softmax scale; 0 => 1/sqrt(128) */
  int32_t policy;             /* KV_POLICY_* */
  int32_t item_tokens;        /* 1 or page_size */
  int32_t dt_steps;           /* decode steps per observation (MemDecay's k) */
  const float *lse_in;        /* [L][Hq][W] natural-log LSE from the attention
                                 backend, or NULL to compute it (extra pass over K) */
  /* MemDecay */
  const uint8_t *region;      /* [N] region label per token (NULL: no regions) */
  const float *base_prio;     /* [n_regions] b_r >= 0 */
  const float *decay_rate;    /* [n_regions] lambda_r >= 0 */
  int32_t n_regions;          /* 1..32; labels are expected below n_regions */
  float rho, alpha, tau;
  float *ewma;                /* [N] in/out (MEMDECAY) */
  int32_t *clock;             /* [N] in/out (MEMDECAY) */
  /* H2O */
  float *accum;               /* [N] in/out (H2O) */
  /* foresight */
  const int32_t *span_id;     /* [N] span of each token, -1 = none (NULL: no bonus) */
  const float *span_bonus;    /* [n_spans] bonus of each span, finite */
  int32_t n_spans;
  /* pinning */
  uint32_t pinned_regions;    /* bit r pins region r */
  int32_t n_sink;
  int32_t n_recent;
  const uint8_t *token_pinned; /* [N] or NULL */
  /* outputs */
  float *mass;                /* [N] mass_j as defined above, or NULL */
  float *lse;                 /* [L][Hq][W] natural-log LSE, or NULL */
  float *token_score;         /* [N] or NULL */
  float *item_score;          /* [ceil(N/item_tokens)] */
  uint8_t *item_pinned;       /* [ceil(N/item_tokens)] */
  /* profiling (optional): host array of 5 events, recorded on the stream before the LSE
     pass, after it, after the LSE combine, after the mass pass and after the epilogue
     (the second and third mark the same point when the mass pass combines the LSE
     itself, which a grid of at most 512 mass-pass workgroups over at most 16 key chunks
     does) */
  hipEvent_t *stage_events;
  int32_t aggregate;          /* KV_AGG_*; memset-zeroed params select KV_AGG_SUM */
  uint32_t *status;           /* device word or NULL: set to 0, then KV_STATUS_BAD_REGION
                                 when some label is >= n_regions */
} kv_score_params;

int32_t kv_abi_version(void);

/* Text for a return code (static storage; KV_EHIP text includes the last HIP error
 * seen by the calling thread). */
const char *kv_strerror(int32_t code);

/* Host-only.  Workspace bytes kv_score needs for this cache and these parameters. */
int32_t kv_score_workspace_size(const kv_cache_desc *cache, const kv_score_params *p,
                                size_t *bytes /* host */);

/* Score every cached token (CalAttn + policy epilogue).  cache and p are host
 * structs; the arrays they point to are device memory.  Updates ewma/clock or accum in
 * place and writes item_score / item_pinned (and mass, lse when given). */
int32_t kv_score(const kv_cache_desc *cache, const kv_score_params *p, void *workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Host-only.  Workspace bytes kv_select needs for n_items items. */
int32_t kv_select_workspace_size(int64_t n_items, size_t *bytes /* host */);

/*
 * Budget selection (MemDecay, Method; PACE Table 1; ActKV Sec. 3.3 "Eviction").
 * Keeps every pinned item, then the best (budget_items - #pinned) other items in the
 * total order: higher score first, exact ties by lower index, -0.0 == +0.0, NaN last.
 * Writes the kept TOKEN indices in ascending order to keep_tokens (pages expand to
 * their tokens; a partial last page contributes the tokens it has), the number of
 * kept tokens to *n_keep (device int64) and KV_STATUS_* bits to *status (device).
 * item_pinned may be NULL.  keep_capacity is the length of keep_tokens in tokens.
 */
int32_t kv_select(const float *item_score, const uint8_t *item_pinned, int64_t n_items,
                  int32_t item_tokens, int64_t n_tokens, int64_t budget_items,
                  int32_t *keep_tokens, int64_t keep_capacity, int64_t *n_keep,
                  uint32_t *status, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * kv_select without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as kv_select; the selection state, histograms and
 * per-block counts live in a fixed 32 KiB device array of the library (one per GPU, held
 * until the process ends), which covers every n_items (KV_EWORKSPACE if it ever did not).
 * Every call on a GPU uses that GPU's one array: calls that overlap on the same GPU (two
 * streams, or two threads) race and must be serialised by the caller.  Each call clears
 * what it needs before using it.  Allocates nothing.
 */
int32_t kv_select_noalloc(const float *item_score, const uint8_t *item_pinned, int64_t n_items,
                          int32_t item_tokens, int64_t n_tokens, int64_t budget_items,
                          int32_t *keep_tokens, int64_t keep_capacity, int64_t *n_keep,
                          uint32_t *status, hipStream_t stream);

/* Host-only.  Workspace bytes kv_lrfu_update needs for n entries. */
int32_t kv_lrfu_workspace_size(int64_t n, size_t *bytes /* host */);

/*
 * ActKV's attention-aware LRFU keep scores ("ActKV: Efficient LLM Agents through
 * Action-Guided KV Cache Management", Sec. 5.1, Algorithm 1, its keep-score update):
 *   s_j = attn_score[j] * scale (float32; e.g. kv_score's group-maximum mass times
 *         1/(L*Hkv*W) gives the mean over layers, KV heads and action queries);
 *   hit_j: j is in the top-p set, the shortest prefix of the entries in the order
 *         (s descending, index ascending, -0 == +0) whose weight reaches top_p * W, where
 *         a finite s > 0 weighs exactly s (other entries weigh 0 and are never hits), W
 *         is the total weight, and every sum and the comparison are exact (no rounding
 *         of any sum); no hits when top_p * W is 0.  top_p = 1 makes every positive
 *         score a hit;
 *   keep_score[j] <- decay * keep_score[j] + (hit_j ? s_j : 0).
 * New entries enter with keep_score 0 (the caller appends them).  The retained set is
 * then kv_select(keep_score, NULL, ...) (Algorithm 1, its TopK selection).  hit (n bytes, 0/1) may be
 * NULL.  top_p in [0, 1], decay in [0, 1].  Deterministic.
 */
int32_t kv_lrfu_update(const float *attn_score, int64_t n, float scale, float top_p, float decay,
                       float *keep_score, uint8_t *hit, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * In-place tail compaction (ActKV Sec. 7.2, Algorithm 4).  With N = cache.n_tokens,
 * block = cache.page_size, Y = ceil(N/block) and X = ceil(budget/block), the target
 * region is logical slots [start, start + budget) with start = (Y - X)*block.  The kept
 * slots outside it (keep_tokens, ascending) move into its slots that hold no kept
 * entry, d-th source to d-th free slot, both ascending; kept slots inside stay.  K, V
 * (every layer and head) and each meta array (src == dst, indexed by slot, covering
 * Y*block slots) move together; keys are not re-rotated, their positions travel as
 * metadata.  Afterwards every kept entry lies in the last X blocks, and blocks
 * [0, start/block) hold nothing kept.  Sources and destinations are disjoint, so all
 * copies run at once without staging.  n_keep (device, may be NULL = max_keep) is clamped
 * to max_keep.  *start_host receives start.  When more kept entries lie outside the
 * region than it has free slots, only the first ones move and *status (device,
 * nullable) gets KV_STATUS_KEEP_OVERFLOW (0 otherwise).  budget >= N moves nothing.
 */
int32_t kv_compact_tail_inplace(const kv_cache_desc *cache, const int32_t *keep_tokens,
                                const int64_t *n_keep, int64_t max_keep, int64_t budget,
                                const kv_meta_desc *meta /* host array */, int32_t n_meta,
                                int64_t *start_host /* host */, uint32_t *status,
                                hipStream_t stream);

/*
 * Rows a compaction drops, gathered for offload (PACE Sec. 3.4: at every compaction the
 * evicted rows go to pinned host memory).  The evicted tokens are the complement of
 * keep_tokens[0:n_keep) (ascending, n_keep a host count) in [0, src.n_tokens), in
 * ascending order; ranks [first, first + count) of them are copied, K and V of every
 * layer and head, to slots 0..count-1 of dst (a device row of the same layer and head
 * shape, dst.n_tokens >= count, not overlapping src).  evicted_tokens[r] (device,
 * nullable) receives the token index of slot r, and every meta array is gathered the
 * same way (dst[r] = src[token]).  KV_EINVAL when first + count exceeds N - n_keep.
 * keep_tokens must be strictly ascending in [0, N); a rank whose token would fall outside
 * the row because of a malformed list is skipped (its slot and id are not written).
 */
int32_t kv_gather_evicted(const kv_cache_desc *src, const int32_t *keep_tokens, int64_t n_keep,
                          int64_t first, int64_t count, const kv_cache_desc *dst,
                          int32_t *evicted_tokens, const kv_meta_desc *meta /* host array */,
                          int32_t n_meta, hipStream_t stream);

/* Host-only.  Device staging bytes kv_offload_evicted needs for chunks of `chunk` tokens. */
int32_t kv_offload_workspace_size(const kv_cache_desc *src, int64_t chunk, size_t *bytes /* host */);

/*
 * Offload every evicted row to host memory: chunks of `chunk` tokens (Penelope swaps
 * through a 1,024-token buffer) are gathered into the device staging workspace with
 * kv_gather_evicted and copied with asynchronous device-to-host copies on `stream`.
 * host_k and host_v (pinned host memory, bf16) receive layout [L][N - n_keep][Hkv][128];
 * host_tokens (pinned host, nullable) the token indices.  Returns after enqueueing; the
 * host buffers are complete once the stream reaches that point.  Chunks run in stream
 * order; the caller overlaps them with work on other streams.
 */
int32_t kv_offload_evicted(const kv_cache_desc *src, const int32_t *keep_tokens, int64_t n_keep,
                           int64_t chunk, void *host_k, void *host_v, int32_t *host_tokens,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Rows coming back from host memory (the inverse of kv_offload_evicted; PACE Sec. 3.4
 * offloads evicted rows, and "Rethinking KV Cache Eviction for Agentic LLM Serving", Part
 * three, moves segments back from the CPU tier): host rows [host_first, host_first +
 * count) of pinned pools host_k / host_v, layout [L][host_rows][Hkv][128] bf16 (the
 * offload layout with host_rows = N - n_keep), are copied to logical slots slots[r]
 * (device int32, distinct; addressed through dst's block table) of every layer and head of
 * dst.  Chunks of `chunk` rows go host-to-device into the staging workspace
 * (kv_offload_workspace_size(dst, chunk)) and are scattered by a kernel, in stream order
 * on `stream`.  Each meta[m] moves with its row: meta[m].dst[slots[r]] = meta[m].src[r]
 * (src a device array of count elements).  A slot outside [0, dst.n_tokens) is skipped.
 * The host pools must stay valid until the stream reaches this point.
 */
int32_t kv_load_rows(const kv_cache_desc *dst, const int32_t *slots, int64_t count,
                     const void *host_k, const void *host_v, int64_t host_rows, int64_t host_first,
                     int64_t chunk, const kv_meta_desc *meta /* host array */, int32_t n_meta,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Host-only.  Workspace bytes kv_swap_chunked needs: two staging areas of `chunk` rows. */
int32_t kv_swap_workspace_size(const kv_cache_desc *cache, int64_t chunk, size_t *bytes /* host */);

/*
 * Penelope's swap when both tiers are full ("Rethinking KV Cache Eviction for Agentic LLM
 * Serving", Part three): the segment in GPU slots slots[0:count) (device int32, distinct)
 * of `cache` moves to the CPU pool host_k / host_v ([L][host_rows][Hkv][128] bf16, pinned),
 * and the CPU segment in pool rows [in_first, in_first + count) moves into those GPU slots.
 * With no free space on either side, a swap buffer of `chunk` CPU rows from buf_first
 * (1,024 tokens in the paper; disjoint from the incoming rows) is used chunk by chunk, in
 * segment order: the chunk leaving the GPU is written into the buffer, the GPU slots it
 * freed receive the matching chunk from the CPU, and the CPU rows that chunk emptied are
 * the buffer for the next chunk.  out_rows (host, nullable, count entries) receives the
 * pool row of every outgoing row, and *next_buf_first (host, nullable) the first row of
 * the incoming segment's last chunk, which is free afterwards.  Only K and V move;
 * workspace as kv_swap_workspace_size(cache, chunk).
 * The outgoing side (gather, device-to-host) runs on `stream` and the incoming side
 * (host-to-device, scatter) on `in_stream`, so the two directions of the host link can
 * overlap; the library orders them with events it creates and releases itself, waits on
 * `stream` before starting, and makes `stream` wait for the whole swap, so the call
 * behaves as one operation on `stream`.  in_stream == stream runs everything in order on
 * one stream.  The streams must have default priority.
 */
int32_t kv_swap_chunked(const kv_cache_desc *cache, const int32_t *slots, int64_t count,
                        void *host_k, void *host_v, int64_t host_rows, int64_t in_first,
                        int64_t buf_first, int64_t chunk, int64_t *out_rows /* host */,
                        int64_t *next_buf_first /* host */, void *workspace,
                        size_t workspace_bytes, hipStream_t stream, hipStream_t in_stream);

/*
 * Segment eviction from the front of the private history ("Rethinking KV Cache
 * Eviction for Agentic LLM Serving", Part one): keep [0, P) and [P + E', N) where
 * E' = min(ceil(E / block) * block, N - P) frees only whole blocks.  Writes the keep
 * list (ascending) when keep_tokens is not NULL, n_keep to *n_keep_dev when not NULL,
 * and returns n_keep and E' through the host pointers.
 */
int32_t kv_select_segment(int64_t n_tokens, int64_t prefix_len, int64_t evict_tokens,
                          int32_t block, int32_t *keep_tokens, int64_t keep_capacity,
                          int64_t *n_keep_dev, int64_t *n_keep_host /* host */,
                          int64_t *evict_len_host /* host */, hipStream_t stream);

/*
 * Stable in-order gather of the kept tokens into dst, with exact re-rotation of the
 * kept keys (PACE Sec. 3.2, Proposition 1; split-half RoPE, Sec. 3.5).
 * Rank r < n_keep takes source token j = keep_tokens[r]:
 *   new_pos[r] = renumber_base + r     when renumber_base >= 0 (order-preserving,
 *                                      gap-collapsing renumbering),
 *              = old_pos[j]            otherwise;
 *   V: copied verbatim;  K: copied verbatim when new_pos[r] == old_pos[j], otherwise
 *   each pair (x_i, x_{i+64}) is rotated by (new_pos[r]-old_pos[j]) * theta_i with
 *   theta_i = rope_theta^(-2i/128), computed in float64 and rounded once to bf16 (RNE).
 *   Every meta[m] array is gathered the same way.
 * n_keep (device, may be NULL = max_keep) is clamped to max_keep (host bound that
 * sizes the launch).  keep_tokens must be ascending indices of src; a rank whose entry
 * lies outside [0, src.n_tokens) is skipped (nothing read or written for it).  dst must
 * not overlap src, and new_pos and the meta destinations must not overlap old_pos,
 * keep_tokens or the meta sources.  KV_EINVAL when they visibly do: K/V extents of
 * caches without a block table, positions and metadata arrays are checked on the host.  dst.n_tokens >= max_keep; its layer and head
 * shapes must equal src's.  limit > 0 with renumbering requires
 * renumber_base + max_keep <= limit (PACE's L), else KV_ELIMIT.  new_pos may be NULL.
 */
int32_t kv_compact_rerope(const kv_cache_desc *src, const kv_cache_desc *dst,
                          const int32_t *keep_tokens, const int64_t *n_keep,
                          int64_t max_keep, const int32_t *old_pos, int32_t *new_pos,
                          int32_t renumber_base, double rope_theta, int32_t limit,
                          const kv_meta_desc *meta /* host array */, int32_t n_meta,
                          hipStream_t stream);

/*
 * RoPE frequency tables (PACE Sec. 3.5: split-half RoPE with static frequency scaling,
 * default, linear, YaRN and Llama-3 style).  theta_i (i < 64) rotates pair (i, i + 64);
 * f_i = base^(-2i/128) is the unscaled frequency and L = original_max_position.
 *   KV_ROPE_DEFAULT: theta_i = f_i
 *   KV_ROPE_LINEAR:  theta_i = f_i / factor
 *   KV_ROPE_LLAMA3:  with w_i = 2 pi / f_i: w_i < L/high_freq_factor keeps the frequency,
 *                    w_i > L/low_freq_factor divides it by factor, in between
 *                    (1-t)/factor + t times it, t = (L/w_i - low_freq_factor) /
 *                    (high_freq_factor - low_freq_factor)
 *   KV_ROPE_YARN:    YaRN's "NTK-by-parts" in the form engines cache keys with: the pair
 *                    turning beta times over L is i(beta) = 128 ln(L/(2 pi beta)) / (2 ln base);
 *                    lo = floor(i(beta_fast)), hi = ceil(i(beta_slow)) (no rounding with
 *                    KV_ROPE_YARN_NO_TRUNCATE), clamped to [0, 127], hi = lo + 0.001 if
 *                    equal; g_i = clamp((i - lo)/(hi - lo), 0, 1) and
 *                    theta_i = g_i f_i / factor + (1 - g_i) f_i
 *   KV_ROPE_YARN_RATIO: the same blend written over r_i = L / w_i as the YaRN paper states
 *                    it: g = clamp((r_i - beta_slow)/(beta_fast - beta_slow), 0, 1),
 *                    theta_i = (1-g) f_i / factor + g f_i (differs from KV_ROPE_YARN inside
 *                    the band; use the form the model's keys were rotated with)
 *   KV_ROPE_TABLE:   the caller's 64 frequencies (host array)
 * Only the rotation is applied: a magnitude factor applied when a key was cached (YaRN's
 * attention temperature) stays in it through any re-rotation.
 */
#define KV_ROPE_DEFAULT 0
#define KV_ROPE_LINEAR 1
#define KV_ROPE_LLAMA3 2
#define KV_ROPE_YARN 3
#define KV_ROPE_TABLE 4
#define KV_ROPE_YARN_RATIO 5

#define KV_ROPE_YARN_NO_TRUNCATE 1   /* kv_rope.flags: keep YaRN's band ends unrounded */

typedef struct kv_rope {
  int32_t kind;                 /* KV_ROPE_* */
  int32_t original_max_position;/* L for LLAMA3 and the YARN kinds */
  double base;                  /* rope_theta, > 1 */
  double factor;                /* LINEAR, LLAMA3, YARN kinds: > 0 */
  double low_freq_factor;       /* LLAMA3 */
  double high_freq_factor;      /* LLAMA3, > low_freq_factor */
  double beta_fast, beta_slow;  /* YARN kinds: band ends in turns over L (32 and 1 typical),
                                   beta_fast > beta_slow > 0 */
  const double *inv_freq;       /* host [64], KV_ROPE_TABLE */
  int32_t flags;                /* KV_ROPE_YARN_NO_TRUNCATE or 0 */
  int32_t reserved;
} kv_rope;

/* Host-only.  The 64 frequencies of *rope; KV_EINVAL for an unknown kind or flag or a bad
 * parameter (non-positive factor, base <= 1, non-finite table entry). */
int32_t kv_rope_inv_freq(const kv_rope *rope, double inv_freq[64] /* host */);

/*
 * Reference store of PACE (Sec. 3.2, non-compounding re-rotation): for every slot of a
 * row, a bf16 copy of the key and the position it is valid at.  Element d of KV head h
 * of slot s in layer l sits at k + l*layer_stride + (s*n_kv_heads + h)*128 + d.
 * pos[s] == KV_REF_NONE marks an empty entry.  A compaction given a store:
 *   - uses slot j's entry when it is not empty and the stored key, re-rotated from
 *     pos[j] to the token's current position and rounded to bf16, equals the cached key
 *     (value equality per element); the new key is then the stored key rotated to the
 *     new position (one rounding), and the entry moves with the token;
 *   - otherwise, when the token's position changes, stores the cached key with its
 *     current position before rotating it (the key's first re-rotation);
 *   - otherwise leaves the destination entry empty.
 * Callers empty the entries of slots they reuse (kv_ref_invalidate); a stale entry that
 * was missed fails the check and is replaced.  Device pointers, caller-owned.
 */
#define KV_REF_NONE INT32_MIN

typedef struct kv_ref_store {
  void *k;                      /* bf16 */
  int32_t *pos;                 /* [n_slots] */
  int64_t n_slots;
  int64_t layer_stride;         /* elements, >= n_slots*n_kv_heads*128 when n_layers > 1 */
} kv_ref_store;

/* Empties entries [first, first + count) of the store (pos = KV_REF_NONE). */
int32_t kv_ref_invalidate(const kv_ref_store *ref, int64_t first, int64_t count,
                          hipStream_t stream);

/*
 * kv_compact_rerope with a frequency table and an optional reference store.  rope NULL
 * means KV_ROPE_DEFAULT with base 1e6.  ref_src (indexed by source token, n_slots >=
 * src.n_tokens) and ref_dst (indexed by rank, n_slots >= max_keep) are both given or
 * both NULL, and must not overlap each other or the caches.  ref_dst entries of ranks
 * >= n_keep are not written.
 */
int32_t kv_compact_rerope_ex(const kv_cache_desc *src, const kv_cache_desc *dst,
                             const int32_t *keep_tokens, const int64_t *n_keep,
                             int64_t max_keep, const int32_t *old_pos, int32_t *new_pos,
                             int32_t renumber_base, const kv_rope *rope /* host */,
                             int32_t limit, const kv_meta_desc *meta /* host array */,
                             int32_t n_meta, const kv_ref_store *ref_src /* host */,
                             const kv_ref_store *ref_dst /* host */, hipStream_t stream);

/*
 * In-place form of segment eviction + compaction + re-rotation: removes tokens
 * [P, P + E') of the row and shifts the suffix [P + E', N) left by E' inside the same
 * cache, re-rotating each moved key by its position change.  pos[N] holds the physical
 * positions on entry; on return pos[0 .. N-E') holds the new ones (renumber_base >= 0:
 * base + r; otherwise unchanged, i.e. Penelope keeps original positions).  The move runs
 * in rounds of at most E' tokens so that no round reads a slot another round of it
 * writes.  Metadata arrays (meta[m].src == meta[m].dst) move the same way.
 */
int32_t kv_compact_segment_inplace(const kv_cache_desc *cache, int64_t prefix_len,
                                   int64_t evict_len, int32_t *pos, int32_t renumber_base,
                                   double rope_theta, int32_t limit,
                                   const kv_meta_desc *meta /* host array */,
                                   int32_t n_meta, hipStream_t stream);

/* kv_compact_segment_inplace with a frequency table (NULL: default, base 1e6) and an
 * optional reference store (n_slots >= N) that moves in place with its tokens.  A token
 * that keeps both its slot and its position is not touched, and neither is its entry. */
int32_t kv_compact_segment_inplace_ex(const kv_cache_desc *cache, int64_t prefix_len,
                                      int64_t evict_len, int32_t *pos, int32_t renumber_base,
                                      const kv_rope *rope /* host */, int32_t limit,
                                      const kv_meta_desc *meta /* host array */, int32_t n_meta,
                                      const kv_ref_store *ref /* host */, hipStream_t stream);

/*
 * Page-table form of segment eviction for a paged cache (cache->block_table != NULL).
 * Penelope frees the evicted segment's blocks ("Rethinking KV Cache Eviction for Agentic
 * LLM Serving", Part one; E' is whole blocks, as kv_select_segment gives); here the
 * surviving suffix is relinked instead of moved.  prefix_len (P) and evict_len (E') must
 * be multiples of page_size.
 *   block_table_out[0 .. ceil((N-E')/page_size))  the new logical->physical map: the
 *       prefix's entries, then the suffix's (logical token r takes the slot of old token
 *       r < P ? r : r + E');
 *   freed_pages[0 .. E'/page_size)  the evicted segment's physical pages (or NULL);
 *   new_pos[r] = renumber_base + r when renumber_base >= 0, else old_pos[source]; a key
 *       whose position changes is re-rotated in place (PACE Sec. 3.2, Proposition 1);
 *       values and unchanged keys are not touched at all;
 *   meta[m].dst[r] = meta[m].src[source] for r < N - E'.
 * Compared with kv_compact_segment_inplace this reads and writes only the keys that
 * change position (nothing at all without renumbering).  Outputs must not overlap any
 * input: block_table_out, freed_pages, new_pos and the metadata destinations are arrays
 * of their own.  limit as in kv_compact_rerope.  No reference store.
 */
int32_t kv_compact_segment_remap(const kv_cache_desc *cache, int64_t prefix_len,
                                 int64_t evict_len, int32_t *block_table_out,
                                 int32_t *freed_pages, const int32_t *old_pos, int32_t *new_pos,
                                 int32_t renumber_base, const kv_rope *rope /* host */,
                                 int32_t limit, const kv_meta_desc *meta /* host array */,
                                 int32_t n_meta, hipStream_t stream);

/*
 * Page-table compaction of a page-mode selection (MemDecay scores pages, S_p, and keeps the
 * best ones; kv_select with item_tokens == page_size writes their tokens as ascending runs
 * of whole pages, the row's partial last page included).  The kept pages are relinked in
 * logical order instead of gathered:
 *   block_table_out[i] = cache->block_table[keep_tokens[i * page_size] / page_size]
 *       for the ceil(n_keep / page_size) kept pages (n_keep: device count, max_keep its
 *       host bound, as for kv_compact_rerope);
 *   new_pos and meta as in kv_compact_rerope; a key whose position changes is re-rotated
 *       in its slot (PACE Sec. 3.2, Proposition 1); values and unchanged keys are not
 *       touched.
 * A kept token that would have to leave its slot (a keep list that is not whole pages) is
 * left alone and sets KV_STATUS_NOT_WHOLE_PAGES in *status (device word or NULL; set to 0
 * otherwise).  The pages no entry of block_table_out names are free; the caller holds both
 * tables.  Outputs must not overlap any input.  No reference store.
 */
int32_t kv_compact_pages_remap(const kv_cache_desc *cache, const int32_t *keep_tokens,
                               const int64_t *n_keep, int64_t max_keep, int32_t *block_table_out,
                               const int32_t *old_pos, int32_t *new_pos, int32_t renumber_base,
                               const kv_rope *rope /* host */, int32_t limit,
                               const kv_meta_desc *meta /* host array */, int32_t n_meta,
                               uint32_t *status, hipStream_t stream);

/* Host-only.  PACE's renumber trigger (Sec. 3.2): 1 when the next physical position
 * comes within headroom of the limit (next_pos >= limit - headroom), else 0. */
int32_t kv_renumber_needed(int64_t next_pos, int32_t headroom, int32_t limit);

#ifdef __cplusplus
}
#endif

#endif /* KVSCORE_H */
