// Internal declarations shared by the HIP translation units of libkvscore.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvscore.h"

namespace kvs {

// KVSCORE_TRACE set (and not "0") in the environment: every launch logs its kernel, grid,
// block and the shape that chose them to stderr, one line each (read once per process).
bool trace_on();
void trace_launch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 128;
constexpr int kTile = 64;          // keys per scoring tile
constexpr int kMaxRows = 512;      // G*W rows per (layer, KV head)
constexpr int kRowsPerGroup = 256; // rows one scoring workgroup covers: 8 waves x 32 rows

// Physical element offset of token j's row start (head 0, dim 0) inside one layer.
__device__ __forceinline__ int64_t token_offset(int64_t j, int page_shift, int64_t page_stride,
                                                const int32_t* __restrict__ block_table,
                                                int slot_stride) {
  const int64_t page = j >> page_shift;
  const int64_t slot = j & ((1LL << page_shift) - 1);
  const int64_t phys = block_table ? (int64_t)block_table[page] : page;
  return phys * page_stride + slot * slot_stride;
}

// ---------------------------------------------------------------- scoring kernels
struct CombineArgs {
  const float2* lse_part;
  int n_chunks, rows, n_kv_heads, n_q_heads, group, window, n_lg, row_stride;
  const float* lse_in;          // optional natural-log LSE input [L][Hq][W]
  float* lse2;                  // [L*Hkv][rows]
  float* lse_out;               // optional [L][Hq][W]
  uint32_t* status;             // optional kv_score status word, cleared here
};

struct ScoreArgs {
  const uint16_t* k;            // bf16 bits
  int64_t layer_stride, page_stride;
  const int32_t* block_table;
  int n_layers, n_kv_heads, page_shift;
  int64_t n_tokens;
  const uint16_t* q;            // bf16 bits [L][W][Hq][128]
  int n_q_heads, window, group, rows;
  int row_stride;               // rows per window query: row = w * row_stride + h_local
  int max_log;                  // 0: sum over query heads; m > 0: max over groups of 2^m rows
  int n_rsplit;                 // workgroups sharing the rows of one (layer, KV head)
  float c;                      // scale * log2(e)
  int chunk, n_chunks;
  float2* lse_part;             // [L*Hkv][n_chunks][rows] (max, sum) in log2 units
  const float* lse2;            // [L*Hkv][rows] log2-unit LSE (pass 2 input)
  float* mass_part;             // [L*Hkv][n_rsplit][N]
  int fuse_combine;             // pass 2 combines its rows' LSE itself (no combine launch)
  CombineArgs comb;             // what that combine reads and writes
};

hipError_t launch_score_pass(const ScoreArgs& a, bool pass2, hipStream_t s);

hipError_t launch_lse_combine(const CombineArgs& a, hipStream_t s);

struct EpilogueArgs {
  const float* mass_part;       // [n_parts][N]
  int n_parts;
  int64_t n_tokens;
  double mass_norm;             // 1 / (L*Hq*W), or 1 / (L*Hkv*W) for the group maximum
  int policy, item_shift;       // item_tokens = 1 << item_shift
  int dt_steps;
  const uint8_t* region;
  const float* base_prio;
  const float* decay_rate;
  int n_regions;
  float rho, alpha, tau;
  float* ewma;
  int32_t* clock;
  float* accum;
  const int32_t* span_id;
  const float* span_bonus;
  int n_spans;
  uint32_t pinned_regions;
  int64_t n_sink, n_recent;
  const uint8_t* token_pinned;
  float* mass;
  float* token_score;
  float* item_score;
  uint8_t* item_pinned;
  uint32_t* status;             // optional: KV_STATUS_BAD_REGION
};
hipError_t launch_epilogue(const EpilogueArgs& a, hipStream_t s);

// ---------------------------------------------------------------- selection kernels
struct SelectState {               // lives in the select workspace
  uint32_t prefix;               // key bits fixed so far
  uint32_t mask;
  int64_t k_rem;                 // items still to take among candidates
  int64_t n_pinned;
  int64_t n_cand;
  uint32_t mode;                 // 0 radix, 1 keep all unpinned, 2 keep none
  uint32_t nan_seen;
  uint32_t ticket;
  uint32_t pad;
};
struct SelectArgs {
  const float* score;
  const uint8_t* pinned;
  int64_t n_items;
  int item_tokens;
  int64_t n_tokens;
  int64_t budget;
  int32_t* keep;
  int64_t keep_capacity;
  int64_t* n_keep;
  uint32_t* status;
  SelectState* st;
  uint32_t* hist;                // [3 passes][kSelBins], cleared by the init kernel
  int64_t* counts;               // [n_blocks][2]
  int n_blocks;
  int64_t per_block;             // items per block
};
constexpr int kSelBins = 2048;     // radix-select histogram bins (11-bit digits)
int select_blocks(int64_t n_items);
size_t select_workspace_bytes(int64_t n_items);
// Fixed per-device scratch that replaces the workspace in kv_select_noalloc.
constexpr size_t kSelectScratchBytes = 32768;
hipError_t select_scratch(void** out);   // this device's address of the scratch array
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_segment_keep(int64_t n_tokens, int64_t prefix, int64_t evict, int32_t* keep,
                               int64_t capacity, int64_t* n_keep_dev, int64_t n_keep,
                               hipStream_t s);

// ---------------------------------------------------------------- LRFU keep scores
struct ToppState {                 // lives in the LRFU workspace
  uint32_t prefix;               // bits of the boundary score fixed so far
  uint32_t mask;
  uint32_t mode;                 // 0 radix, 2 no hits
  uint32_t ticket;
  uint32_t pad0, pad1;
  uint64_t rem;                  // weight still missing from the target, in units of the
                                 // boundary exponent's 2^(E-150)
  int64_t c_eq;                  // entries equal to the boundary that are hits
};
struct LrfuArgs {
  const float* score;            // AttnScore before scaling
  float scale;
  int64_t n;
  float top_p, decay;
  float* keep_score;             // in/out
  uint8_t* hit;                  // nullable
  ToppState* st;
  unsigned long long* hist;      // [3 passes][2048], cleared by the init kernel
  int64_t* counts;               // [n_blocks]
  int n_blocks;
  int64_t per_block;
};
int lrfu_blocks(int64_t n);
size_t lrfu_workspace_bytes(int64_t n);
hipError_t launch_lrfu(const LrfuArgs& a, hipStream_t s);

// ---------------------------------------------------------------- compaction kernels
struct MetaSet {
  const void* src[KV_MAX_META];
  void* dst[KV_MAX_META];
  int elem_bytes[KV_MAX_META];
  int n;
};
struct CompactArgs {
  const uint16_t* src_k;
  const uint16_t* src_v;
  int64_t src_layer_stride, src_page_stride;
  const int32_t* src_bt;
  uint16_t* dst_k;
  uint16_t* dst_v;
  int64_t dst_layer_stride, dst_page_stride;
  const int32_t* dst_bt;
  int n_layers, n_kv_heads, src_page_shift, dst_page_shift;
  int64_t src_tokens;            // tokens of the source row: keep entries outside are skipped
  // rank -> source token: keep[r] when keep != nullptr, else r (+ shift when r >= split)
  const int32_t* keep;
  int64_t split, shift;
  int64_t rank0, rank1;          // ranks handled by this launch
  int parts;                     // workgroups per rank, each moving a contiguous share of its items
  const int64_t* n_keep;         // device count (nullable); ranks >= it are skipped
  const int32_t* old_pos;        // [N] indexed by source token
  int32_t* new_pos;              // [ranks] (nullable)
  int32_t renumber_base;
  double inv_freq[kHeadDim / 2]; // RoPE frequency of pair (i, i + 64)
  // reference store (nullable): keys [L][slot][Hkv][128] bf16 and valid positions [slot]
  const uint16_t* ref_src_k;
  const int32_t* ref_src_pos;
  int64_t ref_src_layer_stride;
  uint16_t* ref_dst_k;
  int32_t* ref_dst_pos;
  int64_t ref_dst_layer_stride;
  MetaSet meta;
  // new_pos and the metadata destinations are the position and metadata sources
  // themselves (the in-place segment form): a rank that keeps its slot and its
  // position then has nothing to write at all
  int rows_in_place;
  // the relinking forms: every rank must already sit in its destination slot; one that
  // does not is left alone and sets KV_STATUS_NOT_WHOLE_PAGES in *status (nullable)
  int remap_only;
  uint32_t* status;
};
// Workgroups per rank that give every thread of the copy at most one item.
int compact_parts(int n_layers, int n_kv_heads);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_ref_invalidate(int32_t* pos, int64_t count, hipStream_t s);
// Page-table form of segment eviction: bt_out[p] = bt[p < prefix_pages ? p : p +
// evict_pages] for p < keep_pages, freed[i] = bt[prefix_pages + i] (nullable).
hipError_t launch_remap_table(const int32_t* bt, int32_t* bt_out, int32_t* freed, int64_t keep_pages,
                              int64_t prefix_pages, int64_t evict_pages, hipStream_t s);
// new_pos[r] = old_pos[source] and the metadata of ranks [0, n), nothing else.
hipError_t launch_remap_rows(const CompactArgs& a, int64_t n, hipStream_t s);
// Page-list form: bt_out[i] = bt[keep[i * page] / page] for the kept pages of
// min(*n_keep, max_keep) kept tokens; *status = 0 (nullable).
hipError_t launch_remap_pages(const int32_t* bt, int32_t* bt_out, const int32_t* keep, const int64_t* n_keep,
                              int64_t max_keep, int page_shift, int64_t n_pages_src, uint32_t* status,
                              hipStream_t s);

struct TailArgs {
  uint16_t* k;
  uint16_t* v;
  int64_t layer_stride, page_stride;
  const int32_t* bt;
  int n_layers, n_kv_heads, page_shift;
  const int32_t* keep;           // ascending kept slots
  const int64_t* n_keep;         // device count (nullable: max_keep)
  int64_t max_keep;
  int64_t n_tokens;              // used slots: keep entries outside [0, n_tokens) are skipped
  int64_t start, budget;         // target region [start, start + budget)
  uint32_t* status;              // nullable
  MetaSet meta;                  // arrays moved in place (src == dst)
};
hipError_t launch_tail_compact(const TailArgs& a, int64_t pairs, hipStream_t s);

struct EvictArgs {
  const uint16_t* src_k;
  const uint16_t* src_v;
  int64_t src_layer_stride, src_page_stride;
  const int32_t* src_bt;
  int src_page_shift;
  uint16_t* dst_k;
  uint16_t* dst_v;
  int64_t dst_layer_stride, dst_page_stride;
  const int32_t* dst_bt;
  int dst_page_shift;
  int n_layers, n_kv_heads;
  const int32_t* keep;           // ascending kept tokens
  int64_t n_keep;
  int64_t src_tokens;            // rows whose token falls outside [0, src_tokens) are skipped
  int64_t first, count;          // evicted ranks [first, first + count)
  int32_t* evicted_tokens;       // [count] (nullable)
  MetaSet meta;                  // dst[e - first] = src[token]
  int parts;                     // workgroups per evicted token (set by the launcher)
};
hipError_t launch_gather_evicted(const EvictArgs& a, hipStream_t s);

// Whole token rows (K and V of every layer and head) between two caches:
// row r copies source token (src_rows ? src_rows[r] : src_first + r) to destination token
// (dst_rows ? dst_rows[r] : dst_first + r); a row whose token lies outside either cache is
// skipped.  meta: dst[dst token] = src[meta_first + r].
struct MoveArgs {
  const uint16_t* src_k;
  const uint16_t* src_v;
  int64_t src_layer_stride, src_page_stride;
  const int32_t* src_bt;
  int src_page_shift;
  int64_t src_tokens;
  uint16_t* dst_k;
  uint16_t* dst_v;
  int64_t dst_layer_stride, dst_page_stride;
  const int32_t* dst_bt;
  int dst_page_shift;
  int64_t dst_tokens;
  int n_layers, n_kv_heads;
  const int32_t* src_rows;
  const int32_t* dst_rows;
  int64_t src_first, dst_first, meta_first;
  int64_t count;
  MetaSet meta;
  int parts;                     // workgroups per row (set by the launcher)
};
hipError_t launch_move_rows(const MoveArgs& a, hipStream_t s);

}  // namespace kvs
