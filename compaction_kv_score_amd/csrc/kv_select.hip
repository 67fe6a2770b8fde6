// Budget selection on gfx950: deterministic radix select with an index tie-break.
//
// MemDecay (Method) keeps pinned tokens unconditionally and fills the rest of a fixed
// budget by score; PACE (Table 1) always keeps 4 sinks and 128 recent tokens; ActKV
// (Sec. 3.3) turns scores and a budget into a keep mask.  Here the kept set is
//   pinned  U  the best (budget - #pinned) unpinned items
// in the total order (score descending, index ascending; -0 == +0; NaN last), and it is
// emitted as an ascending list of token indices so that compaction preserves order.
//
// Steps, all on the device (no host synchronisation; n_keep stays in device memory):
//   1. three histogram passes over 11-, 11- and 10-bit digits of an order-preserving
//      uint32 key, most significant first.  Each block builds a private LDS histogram of
//      the candidates that still match the digits fixed so far and adds it into the
//      pass's global histogram with integer atomics (exact, so the order of the blocks
//      does not matter); the last block to finish (atomic ticket) reads the 2,048 bins
//      and fixes the next digit.
//      Afterwards T is the key of the K-th best unpinned item and k_rem is how many
//      items with key == T are still to be taken (the lowest indices win).
//   2. a count pass: per block, items kept for sure and items equal to T.
//   3. an emit pass: every block derives its output offset from the counts of the
//      blocks before it, then walks its items in index order with wavefront ballots and
//      an LDS scan across waves, and writes the kept token indices.
// A row of at most 4,096 items fits one block: then one launch does the same steps with
// the histograms in LDS and no count pass (there are no other blocks to count); a row of
// at most 256 items finds T and k_rem by counting, for each candidate, the candidates
// ahead of it in the order.

#include <atomic>

#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxBlocks = 64;
constexpr int kWaves = kSelThreads / 64;
constexpr int kBins = kSelBins;
// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt not waited for
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s) return 0u;                 // NaN orders after every number
  if (u == 0x80000000u) u = 0u;          // -0.0 counts as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool item_pinned(const SelectArgs& a, int64_t i) {
  return a.pinned != nullptr && a.pinned[i] != 0;
}

// Items a thread loads before it processes any of them: the loads of a batch are all in
// flight together instead of one memory round trip per item.
constexpr int kSelBatch = 4;

// Rows of at most this many items rank their candidates by counting in the one-block
// kernel (a few hundred comparisons per thread) instead of three histogram passes.
constexpr int kRankItems = 256;

// Score and pinned flag of items b0 + u*kSelThreads + tid (u < kSelBatch) before `end`.
__device__ __forceinline__ void load_batch(const SelectArgs& a, int64_t b0, int64_t end,
                                           float (&sc)[kSelBatch], bool (&pin)[kSelBatch]) {
#pragma unroll
  for (int u = 0; u < kSelBatch; ++u) {
    const int64_t i = b0 + (int64_t)u * kSelThreads + threadIdx.x;
    const bool in = i < end;
    pin[u] = in && item_pinned(a, i);
    sc[u] = in ? a.score[i] : 0.f;
  }
}

// Add 1 to bin[d] for every lane with `want`.  Scores of a long row are concentrated in
// a few bins, so the lanes sharing the most common digits are merged into one atomic
// each first and only the rest are added one by one.
__device__ __forceinline__ void hist_add(uint32_t* bin, bool want, uint32_t d) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const uint64_t act = __builtin_amdgcn_ballot_w64(want);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
    const uint64_t same = __builtin_amdgcn_ballot_w64(want && d == dl);
    if (lane == leader) atomicAdd(&bin[dl], (uint32_t)__popcll(same));
    if (d == dl) want = false;
  }
  if (want) atomicAdd(&bin[d], 1u);
}

// Digit widths of the three MSB-first passes: 11, 11 and 10 bits.
__device__ __forceinline__ int pass_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t pass_dmask(int pass) { return pass == 2 ? 1023u : 2047u; }

// ---- steps shared by the multi-block sequence and the one-block kernel

// Adds the candidates among this block's items [begin, end) to the LDS histogram h for
// one pass (unpinned items whose key matches `prefix` under `mask`), and counts pinned
// items and NaN scores (any item, pinned ones included).  sc/pin hold the first batch.
__device__ __forceinline__ void hist_items(const SelectArgs& a, int64_t begin, int64_t end,
                                           float (&sc)[kSelBatch], bool (&pin)[kSelBatch], int pass,
                                           uint32_t prefix, uint32_t mask, uint32_t* h, uint32_t& npin,
                                           uint32_t& nan_seen) {
  const int shift = pass_shift(pass);
  const uint32_t dmask = pass_dmask(pass);
  for (int64_t b0 = begin; b0 < end; b0 += (int64_t)kSelThreads * kSelBatch) {
    if (b0 != begin) load_batch(a, b0, end, sc, pin);
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const bool in = b0 + (int64_t)u * kSelThreads + threadIdx.x < end;
      const uint32_t key = order_key(sc[u]);
      npin += pin[u] ? 1u : 0u;
      nan_seen |= (in && sc[u] != sc[u]) ? 1u : 0u;
      hist_add(h, in && !pin[u] && (key & mask) == prefix, (key >> shift) & dmask);
    }
  }
}

// The state after pass 0's counts: how many unpinned items are still to be taken, and
// whether the radix passes are needed at all (mode 1: every unpinned item fits; mode 2:
// the pinned items alone fill the budget).
__device__ __forceinline__ void start_state(SelectState& st, const SelectArgs& a, int64_t n_pin, uint32_t nan_any) {
  st.n_pinned = n_pin;
  st.n_cand = a.n_items - n_pin;
  st.nan_seen = nan_any;
  st.prefix = 0;
  st.mask = 0;
  const int64_t k = a.budget - n_pin;
  st.k_rem = k;
  st.mode = k >= st.n_cand ? 1u : (k <= 0 ? 2u : 0u);
}

// Block-wide (every thread calls it): from the complete histogram h of a pass, the digit
// at which the count from the top reaches st.k_rem; narrows st (prefix, mask, k_rem).
// Thread t owns bins 2047-2t and 2046-2t (descending); an exclusive scan of the pair
// sums locates the bin.
__device__ __forceinline__ void decide_digit(const uint32_t* h, SelectState& st, int pass, uint32_t* s_wsum) {
  if (st.mode != 0) return;  // uniform: st is shared
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t k_rem = st.k_rem;
  const uint32_t c0 = h[kBins - 1 - 2 * tid], c1 = h[kBins - 2 - 2 * tid];
  uint32_t incl = c0 + c1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wv; ++w) before += s_wsum[w];
  const int64_t excl = before + incl - (c0 + c1);
  int digit = -1;
  int64_t above = 0;
  if (excl < k_rem && excl + c0 >= k_rem) {
    digit = kBins - 1 - 2 * tid;
    above = excl;
  } else if (excl + c0 < k_rem && excl + c0 + c1 >= k_rem) {
    digit = kBins - 2 - 2 * tid;
    above = excl + c0;
  }
  if (digit >= 0) {
    st.k_rem = k_rem - above;
    st.prefix |= (uint32_t)digit << pass_shift(pass);
    st.mask |= pass_dmask(pass) << pass_shift(pass);
  }
  __syncthreads();
}

// Exclusive prefixes of two per-thread flags over the block in one pass (per-wave
// counts packed as a | b << 16, at most 64 each).
__device__ __forceinline__ void block_scan2(bool fa, bool fb, uint32_t* s_wave, uint32_t& ra, uint32_t& rb,
                                            uint32_t& ta, uint32_t& tb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const uint64_t ba = __builtin_amdgcn_ballot_w64(fa);
  const uint64_t bb = __builtin_amdgcn_ballot_w64(fb);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) s_wave[wv] = (uint32_t)__popcll(ba) | ((uint32_t)__popcll(bb) << 16);
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = s_wave[w];
    before += w < wv ? c : 0u;
    tot += c;
  }
  __syncthreads();
  ra = (before & 0xFFFFu) + (uint32_t)__popcll(ba & below);
  rb = (before >> 16) + (uint32_t)__popcll(bb & below);
  ta = tot & 0xFFFFu;
  tb = tot >> 16;
}

// Writes the kept token indices of items [begin, end) in index order, given the items
// kept before `begin` and the ties (key == T) before it; returns the items kept up to
// `end`.  Sets *s_last_kept when the row's last item is kept.  sc/pin hold the first batch.
__device__ __forceinline__ int64_t emit_items(const SelectArgs& a, int64_t begin, int64_t end,
                                              float (&sc)[kSelBatch], bool (&pin)[kSelBatch], uint32_t mode,
                                              uint32_t T, int64_t k_rem, int64_t kept_before, int64_t eq_before,
                                              uint32_t* s_wave, int* s_last_kept) {
  const int tid = threadIdx.x;
  const int it = a.item_tokens;
  for (int64_t base = begin; base < end; base += kSelThreads) {
    const int u = (int)(((base - begin) / kSelThreads) % kSelBatch);
    if (base != begin && u == 0) load_batch(a, base, end, sc, pin);
    const int64_t i = base + tid;
    const bool valid = i < end;
    bool def = false, eq = false;
    float sc_u = sc[0];
    bool pin_u = pin[0];
#pragma unroll
    for (int v = 1; v < kSelBatch; ++v)
      if (u == v) {
        sc_u = sc[v];
        pin_u = pin[v];
      }
    if (valid) {
      if (pin_u || mode == 1u) {
        def = true;
      } else if (mode == 0u) {
        const uint32_t key = order_key(sc_u);
        def = key > T;
        eq = key == T;
      }
    }
    // def and eq are exclusive; the first max(0, k_rem - eq_before) ties of this round
    // (in index order) are taken, so one scan of both flags gives every output rank
    uint32_t def_rank, eq_rank, def_total, eq_total;
    block_scan2(def, eq, s_wave, def_rank, eq_rank, def_total, eq_total);
    const int64_t ties_left = k_rem - eq_before > 0 ? k_rem - eq_before : 0;
    const bool kept = def || (eq && (int64_t)eq_rank < ties_left);
    const uint32_t out_rank = def_rank + (uint32_t)((int64_t)eq_rank < ties_left ? eq_rank : ties_left);
    const uint32_t kept_total =
        def_total + (uint32_t)((int64_t)eq_total < ties_left ? eq_total : ties_left);
    if (kept) {
      const int64_t out = (kept_before + out_rank) * it;
      const int64_t t0 = i * it;
      const int64_t t1 = t0 + it < a.n_tokens ? t0 + it : a.n_tokens;
      for (int64_t t = t0; t < t1; ++t) {
        const int64_t o = out + (t - t0);
        if (o < a.keep_capacity) a.keep[o] = (int32_t)t;
      }
      if (i == a.n_items - 1) *s_last_kept = 1;
    }
    kept_before += kept_total;
    eq_before += eq_total;
  }
  return kept_before;
}

// One thread: the kept token count and the status word of the row.
__device__ __forceinline__ void write_result(const SelectArgs& a, int64_t kept_items, bool last_kept,
                                             uint32_t nan_seen, int64_t n_pinned) {
  // the last item may be a partial page holding n_tokens - (n_items-1)*it tokens
  const int it = a.item_tokens;
  int64_t n_tok = kept_items * it;
  if (last_kept) n_tok -= (int64_t)a.n_items * it - a.n_tokens;
  *a.n_keep = n_tok;
  uint32_t status = 0;
  if (nan_seen) status |= KV_STATUS_NAN_SCORE;
  if (n_pinned > a.budget) status |= KV_STATUS_PINNED_OVER_BUDGET;
  if (n_tok > a.keep_capacity) status |= KV_STATUS_KEEP_OVERFLOW;
  if (a.status) *a.status = status;
}

// ---- the multi-block sequence

__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelectArgs a, int pass) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t s_wsum[kWaves];
  __shared__ uint32_t s_npin, s_nan;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n_items ? begin + a.per_block : a.n_items;
  // the first batch is requested before the state, so the two latencies overlap
  float sc[kSelBatch];
  bool pin[kSelBatch];
  load_batch(a, begin, end, sc, pin);
  const uint32_t mode = pass == 0 ? 0u : a.st->mode;
  const uint32_t prefix = pass == 0 ? 0u : a.st->prefix;
  const uint32_t mask = pass == 0 ? 0u : a.st->mask;
  for (int b = tid; b < kBins; b += kSelThreads) h[b] = 0;
  if (tid == 0) {
    s_npin = 0;
    s_nan = 0;
  }
  __syncthreads();
  if (mode != 0) return;  // decided without a radix pass (uniform across the grid)

  uint32_t npin = 0, nan_seen = 0;
  hist_items(a, begin, end, sc, pin, pass, prefix, mask, h, npin, nan_seen);
  if (pass == 0) {
    if (npin) atomicAdd(&s_npin, npin);
    if (nan_seen) atomicOr(&s_nan, 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)pass * kBins;
  for (int b = tid; b < kBins; b += kSelThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
  if (pass == 0 && tid == 0) {
    a.counts[2 * blockIdx.x] = s_npin;
    a.counts[2 * blockIdx.x + 1] = s_nan;
  }
  // Every wave waits for its own histogram atomics to complete; then one thread makes
  // the block's results visible device-wide (the release writes back the whole L2, so
  // one per block suffices: one per wave cost ~7 us per pass) and takes the ticket.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    __builtin_amdgcn_s_waitcnt(kVmcntZero);   // the write-back has completed
    s_last = atomicAdd(&a.st->ticket, 1u) == (uint32_t)gridDim.x - 1u;
  }
  __syncthreads();
  if (!s_last) return;
  // acquire for wave 0, the only wave that reads shared data through the caches (the
  // histograms below are read with cache-bypassing atomic loads)
  if (threadIdx.x < 64) __threadfence();

  // ---- last block: the global histogram of this pass, then the digit
  const int nb = (int)gridDim.x;
  for (int b = tid; b < kBins; b += kSelThreads) h[b] = __atomic_load_n(&gh[b], __ATOMIC_RELAXED);
  __shared__ SelectState st;
  if (wv == 0) {
    // pass 0: lane b reads block b's counts (at most 64 blocks), then a wave-wide sum
    int64_t n_pin = 0;
    uint32_t nan_any = 0;
    if (pass == 0) {
      if (lane < nb) {
        n_pin = __atomic_load_n(&a.counts[2 * lane], __ATOMIC_RELAXED);
        nan_any = (uint32_t)__atomic_load_n(&a.counts[2 * lane + 1], __ATOMIC_RELAXED);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        n_pin += __shfl_xor(n_pin, off);
        nan_any |= __shfl_xor(nan_any, off);
      }
    }
    if (lane == 0) st = *a.st;
    if (lane == 0 && pass == 0) start_state(st, a, n_pin, nan_any);
  }
  __syncthreads();
  decide_digit(h, st, pass, s_wsum);
  if (tid == 0) {
    st.ticket = 0;
    *a.st = st;
    __threadfence();
  }
}

// Per block: items kept for sure (pinned, or key above T, or everything in mode 1) and
// unpinned items whose key equals T (ties, resolved by index in the emit pass).
__global__ __launch_bounds__(kSelThreads) void select_count_kernel(SelectArgs a) {
  __shared__ uint32_t s_def, s_eq;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_def = 0;
    s_eq = 0;
  }
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n_items ? begin + a.per_block : a.n_items;
  float sc[kSelBatch];
  bool pin[kSelBatch];
  load_batch(a, begin, end, sc, pin);
  const uint32_t mode = a.st->mode;
  const uint32_t T = a.st->prefix;
  __syncthreads();
  uint32_t def = 0, eq = 0;
  for (int64_t b0 = begin; b0 < end; b0 += (int64_t)kSelThreads * kSelBatch) {
    if (b0 != begin) load_batch(a, b0, end, sc, pin);
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      if (b0 + (int64_t)u * kSelThreads + tid >= end) continue;
      if (pin[u] || mode == 1u) {
        ++def;
        continue;
      }
      if (mode == 2u) continue;
      const uint32_t key = order_key(sc[u]);
      def += key > T;
      eq += key == T;
    }
  }
  if (def) atomicAdd(&s_def, def);
  if (eq) atomicAdd(&s_eq, eq);
  __syncthreads();
  if (tid == 0) {
    a.counts[2 * blockIdx.x] = s_def;
    a.counts[2 * blockIdx.x + 1] = s_eq;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_emit_kernel(SelectArgs a) {
  __shared__ uint32_t s_wave[kWaves];
  __shared__ int64_t s_kept_before, s_eq_before;
  __shared__ int s_last_kept;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n_items ? begin + a.per_block : a.n_items;
  float sc[kSelBatch];
  bool pin[kSelBatch];
  load_batch(a, begin, end, sc, pin);
  const uint32_t mode = a.st->mode;
  const uint32_t T = a.st->prefix;
  const int64_t k_rem = mode == 0u ? a.st->k_rem : 0;
  if (tid < 64) {
    // lane b holds block b's counts (b < blockIdx.x <= 63); ties are taken in block order,
    // so block b takes clamp(k_rem - ties of blocks before b, 0, its ties)
    const bool mine = lane < (int)blockIdx.x;
    const int64_t def = mine ? a.counts[2 * lane] : 0;
    const int64_t eq = mine ? a.counts[2 * lane + 1] : 0;
    int64_t eq_incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t v = __shfl_up(eq_incl, off);
      if (lane >= off) eq_incl += v;
    }
    int64_t take = k_rem - (eq_incl - eq);
    take = take < 0 ? 0 : (take > eq ? eq : take);
    int64_t kept = def + take;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kept += __shfl_xor(kept, off);
    const int64_t eqb = __shfl(eq_incl, 63);
    if (lane == 0) {
      s_kept_before = kept;
      s_eq_before = eqb;
      s_last_kept = 0;
    }
  }
  __syncthreads();
  const int64_t kept = emit_items(a, begin, end, sc, pin, mode, T, k_rem, s_kept_before, s_eq_before, s_wave,
                                  &s_last_kept);
  __syncthreads();
  if (blockIdx.x == gridDim.x - 1 && tid == 0) write_result(a, kept, s_last_kept != 0, a.st->nan_seen, a.st->n_pinned);
}

// ---- rows that fit one block (at most kSelThreads * kSelBatch items): every step in one
// launch.  Each thread loads its items once; the three passes build their histograms in
// LDS, the digits are decided in place, and the emit needs no counts of other blocks.
// No workspace memory is touched.
__global__ __launch_bounds__(kSelThreads) void select_one_block_kernel(SelectArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t s_wave[kWaves];
  __shared__ uint32_t s_npin, s_nan;
  __shared__ int s_last_kept;
  __shared__ SelectState st;
  const int tid = threadIdx.x;
  float sc[kSelBatch];
  bool pin[kSelBatch];
  load_batch(a, 0, a.n_items, sc, pin);
  if (tid == 0) {
    s_npin = 0;
    s_nan = 0;
    s_last_kept = 0;
  }
  if (a.n_items <= kRankItems) {
    // A short row: each candidate counts the candidates before it in the order (higher
    // key, or equal key and lower index) instead of three histogram passes; the boundary
    // key T and the ties still to take come out as the passes would give them.  Four
    // neighbouring lanes share an item, each counting a quarter of the row, 4 keys per
    // 16-byte LDS read; two lane swaps add the quarters.
    __shared__ __attribute__((aligned(16))) uint32_t s_key[kRankItems];
    __shared__ __attribute__((aligned(16))) uint32_t s_cand[kRankItems];   // 1 = candidate
    const int n = (int)a.n_items;
    if (tid < kRankItems) {
      const bool in = tid < n;
      s_key[tid] = order_key(sc[0]);
      s_cand[tid] = (in && !pin[0]) ? 1u : 0u;
      if (in && pin[0]) atomicAdd(&s_npin, 1u);
      if (in && sc[0] != sc[0]) atomicOr(&s_nan, 1u);
    }
    __syncthreads();
    if (tid == 0) start_state(st, a, s_npin, s_nan);
    __syncthreads();
    const uint32_t mode0 = st.mode;
    const int64_t k_rem = st.k_rem;
    __syncthreads();   // every thread holds the state before one of them rewrites it
    const int item = tid >> 2, quarter = tid & 3;
    if (mode0 == 0u && item < kRankItems) {                      // uniform per wave
      const uint32_t key = s_key[item];
      const bool cand = s_cand[item] != 0u;
      const int span = ((n + 15) / 16) * 4;                      // keys per quarter, a multiple of 4
      const int j0 = quarter * span;
      uint32_t above = 0, equal = 0, equal_before = 0;
      for (int j = j0; j < j0 + span; j += 4) {
        const uint4 k4 = *(const uint4*)&s_key[j];
        const uint4 c4 = *(const uint4*)&s_cand[j];
        const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
        const uint32_t cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          above += (kk[u] > key) ? cc[u] : 0u;
          const uint32_t eq = (kk[u] == key) ? cc[u] : 0u;
          equal += eq;
          equal_before += (j + u < item) ? eq : 0u;
        }
      }
      above += __shfl_xor(above, 1);
      above += __shfl_xor(above, 2);
      equal += __shfl_xor(equal, 1);
      equal += __shfl_xor(equal, 2);
      equal_before += __shfl_xor(equal_before, 1);
      equal_before += __shfl_xor(equal_before, 2);
      // the first of the candidates with key T writes the state
      if (quarter == 0 && cand && equal_before == 0 && (int64_t)above < k_rem &&
          k_rem <= (int64_t)(above + equal)) {
        st.prefix = key;
        st.mask = 0xFFFFFFFFu;
        st.k_rem = k_rem - above;
      }
    }
    __syncthreads();
  } else {
  for (int pass = 0; pass < 3; ++pass) {
    for (int b = tid; b < kBins; b += kSelThreads) h[b] = 0;
    __syncthreads();   // also closes the previous pass's reads of h and its update of st
    if (pass > 0 && st.mode != 0) break;   // uniform
    uint32_t npin = 0, nan_seen = 0;
    hist_items(a, 0, a.n_items, sc, pin, pass, pass == 0 ? 0u : st.prefix, pass == 0 ? 0u : st.mask, h, npin,
               nan_seen);
    if (pass == 0) {
      if (npin) atomicAdd(&s_npin, npin);
      if (nan_seen) atomicOr(&s_nan, 1u);
    }
    __syncthreads();
    if (pass == 0) {
      if (tid == 0) start_state(st, a, s_npin, s_nan);
      __syncthreads();
    }
    decide_digit(h, st, pass, s_wave);
  }
  }
  const uint32_t mode = st.mode;
  const int64_t kept = emit_items(a, 0, a.n_items, sc, pin, mode, st.prefix, mode == 0u ? st.k_rem : 0, 0, 0,
                                  s_wave, &s_last_kept);
  __syncthreads();
  if (tid == 0) write_result(a, kept, s_last_kept != 0, st.nan_seen, st.n_pinned);
}

__global__ __launch_bounds__(256) void segment_keep_kernel(int64_t prefix, int64_t evict,
                                                           int32_t* keep, int64_t n_write,
                                                           int64_t* n_keep_dev, int64_t n_keep) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r == 0 && n_keep_dev) *n_keep_dev = n_keep;
  if (keep && r < n_write) keep[r] = (int32_t)(r < prefix ? r : r + evict);
}

}  // namespace

// A row that fits one block's batch takes the one-block kernel; larger rows spread over
// blocks of about 2,048 items (at most 64 blocks): the passes are latency bound, and more
// blocks overlap more of it (measured at 100,000 items in the step: 4,096 items per block
// 58.8-59.5 us, 2,048 52.8-53.1 us, 1,563 52.7-53.2 us, 8,192 69.9-70.6 us).
int select_blocks(int64_t n_items) {
  if (n_items <= (int64_t)kSelThreads * kSelBatch) return 1;
  int64_t b = (n_items + 2047) / 2048;
  if (b > kSelMaxBlocks) b = kSelMaxBlocks;
  return (int)b;
}

size_t select_workspace_bytes(int64_t n_items) {
  const int nb = select_blocks(n_items);
  return 256 + (size_t)3 * kBins * sizeof(uint32_t) + (size_t)nb * 2 * sizeof(int64_t);
}

// Clears the selection state and the three pass histograms (a kernel rather than a
// memset, so that the sequence can be captured in a graph).
__global__ __launch_bounds__(kSelThreads) void select_init_kernel(SelectState* st, uint32_t* hist) {
  for (int i = threadIdx.x; i < 3 * kBins; i += kSelThreads) hist[i] = 0;
  if (threadIdx.x == 0) {
    SelectState z;
    memset(&z, 0, sizeof(z));
    *st = z;
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (trace_on())
    trace_launch(a.n_blocks == 1 ? "select one block (3 hist passes, emit) grid=%d block=%d  items=%lld item_tokens=%d budget=%lld"
                                 : "select init+3 hist+count+emit grid=%d block=%d  items=%lld item_tokens=%d budget=%lld",
                 a.n_blocks, kSelThreads, (long long)a.n_items, a.item_tokens, (long long)a.budget);
  if (a.n_blocks == 1) {
    // the whole row fits one block: one launch instead of six
    hipLaunchKernelGGL(select_one_block_kernel, dim3(1), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(select_init_kernel, dim3(1), dim3(kSelThreads), 0, s, a.st, a.hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.n_blocks), block(kSelThreads);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(select_hist_kernel, grid, block, 0, s, a, pass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_count_kernel, grid, block, 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_emit_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

// ---- fixed scratch of kv_select_noalloc
// The selection state, the three pass histograms and the per-block counts of at most
// kSelMaxBlocks blocks (select_workspace_bytes never exceeds 25,856 bytes) in one file-scope
// array per device, for callers that cannot allocate.  Each device holds its own copy at
// its own address; host code only ever uses that address, taken once per device.
static __device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
}  // namespace

hipError_t select_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with this device current: the address of its copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_segment_keep(int64_t n_tokens, int64_t prefix, int64_t evict, int32_t* keep,
                               int64_t capacity, int64_t* n_keep_dev, int64_t n_keep,
                               hipStream_t s) {
  (void)n_tokens;
  const int64_t n_write = keep ? (n_keep < capacity ? n_keep : capacity) : 0;
  const int64_t n = n_write > 1 ? n_write : 1;
  if (trace_on())
    trace_launch("segment_keep grid=%lld block=256  tokens=%lld prefix=%lld evict=%lld", (long long)((n + 255) / 256),
                 (long long)n_tokens, (long long)prefix, (long long)evict);
  hipLaunchKernelGGL(segment_keep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     prefix, evict, keep, n_write, n_keep_dev, n_keep);
  return hipGetLastError();
}

}  // namespace kvs
