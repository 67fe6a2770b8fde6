// ActKV's attention-aware LRFU keep scores (ActKV Sec. 5.1, Algorithm 1) on gfx950.
//
//   KS <- decay * KS + AttnScore   for hits,   KS <- decay * KS   for misses,
// where an entry is a hit when its score lies in the top-p set: the shortest prefix of
// the entries in the total order (score descending, index ascending) whose weight
// reaches p times the total weight.  A finite positive score weighs exactly its value;
// other entries weigh nothing and are never hits.  Every sum is exact:
//   - a finite positive float32 is M * 2^(E-150) with the integer M = 1.mantissa * 2^23
//     (subnormals: M = mantissa, E = 1);
//   - the first radix digit of a score (its top 11 bits) fixes E, so one histogram bin
//     holds scores of a single exponent and its weight is the integer sum of their M;
//   - the last block of the first pass adds the bins as multi-word integers in units of
//     2^-149 (the spacing of the smallest subnormal) and compares them with the target
//     p * W, both exact, to find the boundary bin and what is missing of the target in
//     that bin's units;
//   - from there every candidate shares E, so the later passes are uint64 sums of M.
// The hit set therefore does not depend on the order of any addition.
//
// Steps (no host synchronisation):
//   1. three weighted radix passes over the 11-, 11- and 10-bit digits of the score bits:
//      per-block LDS histograms of weight sums (64-bit integer atomics), added into one
//      global histogram per pass with 64-bit integer atomics; the last block to finish
//      reads it and fixes the digit where the weight counted from the top reaches what is
//      still missing of the target.  Afterwards T is the boundary score and c the
//      number of entries equal to T (lowest indices first) that complete the target;
//   2. a count pass (entries equal to T per block) and an update pass that walks the
//      entries in index order, decides hits and writes KS (and the hit mask).
// A row of at most 4,096 entries fits one block: then one launch does the same steps with
// the state and the histograms in LDS and no count pass.
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 64;
constexpr int kMaxPerBlock = 4096;  // rows up to this size run in one block
constexpr int kPerBlock = 2048;     // entries per block for longer rows, while the grid has room
constexpr int kBins = 2048;
constexpr int kLimbs = 12;          // 384-bit integers: the total weight stays below 2^336
// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt not waited for
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

__device__ __forceinline__ bool has_weight(float s) { return s > 0.f && s <= 3.402823466e38f; }

// M of a finite positive score: the significand as an integer (24 bits at most)
__device__ __forceinline__ uint64_t weight(float s) {
  if (!has_weight(s)) return 0ull;
  const uint32_t b = __float_as_uint(s);
  return (uint64_t)((b & 0x7FFFFFu) | ((b >> 23) != 0 ? 0x800000u : 0u));
}

__device__ __forceinline__ int pass_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t pass_dmask(int pass) { return pass == 2 ? 1023u : 2047u; }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d), hi = __shfl_up((uint32_t)(v >> 32), d);
  return ((uint64_t)hi << 32) | lo;
}

// Add w to bin[d] for every lane with `want`.  Lanes sharing the digit of a leader are
// summed with a wavefront reduction first (scores concentrate in a few bins).
__device__ __forceinline__ void hist_add(unsigned long long* bin, bool want, uint32_t d, uint64_t w) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint64_t act = __builtin_amdgcn_ballot_w64(want);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
    const bool same = want && d == dl;
    uint64_t v = same ? w : 0ull;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor64(v, m);
    if (lane == leader && v) atomicAdd(&bin[dl], (unsigned long long)v);
    if (same) want = false;
  }
  if (want && w) atomicAdd(&bin[d], (unsigned long long)w);
}

// Clears the state and the three pass histograms (a kernel rather than a memset, so that
// the sequence can be captured in a graph).
__global__ __launch_bounds__(kThreads) void lrfu_init_kernel(ToppState* st, unsigned long long* hist) {
  for (int i = threadIdx.x; i < 3 * kBins; i += kThreads) hist[i] = 0ull;
  if (threadIdx.x == 0) {
    ToppState z;
    z.prefix = 0;
    z.mask = 0;
    z.mode = 0;
    z.ticket = 0;
    z.pad0 = 0;
    z.pad1 = 0;
    z.rem = 0;
    z.c_eq = 0;
    *st = z;
  }
}

__device__ __forceinline__ float item_score(const LrfuArgs& a, int64_t i) { return a.score[i] * a.scale; }

// ---- multi-word unsigned integers: kLimbs little-endian 32-bit limbs
struct Big {
  uint32_t l[kLimbs];
};

// Carry-propagate per-limb sums (each below 2^63) into limbs.
__device__ __forceinline__ Big normalize(const uint64_t (&v)[kLimbs]) {
  Big r;
  uint64_t carry = 0;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    const uint64_t x = v[j] + carry;
    r.l[j] = (uint32_t)x;
    carry = x >> 32;
  }
  return r;
}

__device__ __forceinline__ bool big_less(const Big& a, const Big& b) {   // a < b
#pragma unroll
  for (int j = kLimbs - 1; j >= 0; --j)
    if (a.l[j] != b.l[j]) return a.l[j] < b.l[j];
  return false;
}

__device__ __forceinline__ bool big_zero(const Big& a) {
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) o |= a.l[j];
  return o == 0;
}

// a - b for a >= b
__device__ __forceinline__ Big big_sub(const Big& a, const Big& b) {
  Big r;
  int64_t borrow = 0;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    const int64_t x = (int64_t)a.l[j] - (int64_t)b.l[j] - borrow;
    r.l[j] = (uint32_t)x;
    borrow = x < 0 ? 1 : 0;
  }
  return r;
}

// ceil(a / 2^sh) for 0 <= sh < 32 * kLimbs, when the quotient fits in 64 bits
__device__ __forceinline__ uint64_t big_shr_ceil64(const Big& a, int sh) {
  const int q = sh >> 5, r = sh & 31;
  uint64_t out = 0;
  bool sticky = false;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    const uint64_t limb = a.l[j];
    if (j < q) {
      sticky |= limb != 0;
    } else if (j == q) {
      sticky |= r != 0 && (limb & ((1ull << r) - 1ull)) != 0;
      out |= limb >> r;
    } else if (j - q < 3) {
      // limb j lands at bit 32*(j-q) - r of the quotient; bits beyond 63 are zero
      // when the quotient fits in 64 bits
      const int pos = 32 * (j - q) - r;
      if (pos < 64) out |= limb << pos;
    }
  }
  return out + (sticky ? 1ull : 0ull);
}

// ceil(mp * T / 2^k) for a 24-bit mp and 23 <= k < 32 * kLimbs (p = mp * 2^-k <= 1)
__device__ Big topp_target(const Big& T, uint32_t mp, int k) {
  uint32_t x[kLimbs + 1];
  uint64_t carry = 0;
  for (int j = 0; j < kLimbs; ++j) {
    const uint64_t v = (uint64_t)T.l[j] * mp + carry;
    x[j] = (uint32_t)v;
    carry = v >> 32;
  }
  x[kLimbs] = (uint32_t)carry;
  const int q = k >> 5, r = k & 31;
  bool sticky = false;
  for (int j = 0; j < q; ++j) sticky |= x[j] != 0;
  if (r) sticky |= (x[q] & ((1u << r) - 1u)) != 0;
  Big t;
  for (int j = 0; j < kLimbs; ++j) {
    const int src = j + q;
    const uint64_t lo = src <= kLimbs ? x[src] : 0u;
    const uint64_t hi = src + 1 <= kLimbs ? x[src + 1] : 0u;
    t.l[j] = (uint32_t)(((hi << 32) | lo) >> r);
  }
  if (sticky) {
    for (int j = 0; j < kLimbs; ++j) {
      if (++t.l[j] != 0) break;
    }
  }
  return t;
}

// Pass 0, last block: finds the boundary bin of the exact top-p set.  Thread t < 256
// owns exponent E = 255 - t (descending), i.e. bins 4E..4E+3 (bins >= 1024 hold no
// positive score), whose weight is Y = sum of M times 2^(max(E,1) - 1) units of 2^-149.
// A scan over the threads gives every exponent's cumulative weight from the top as an
// exact multi-word integer; the target is ceil(p * W) in the same units (the prefix
// weight is an integer, so reaching p * W is reaching its ceiling).
__device__ void topp_first_digit(const unsigned long long* h, float top_p, ToppState& st,
                                 uint64_t (*s_wtot)[kLimbs], Big& s_total, Big& s_target) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = 255 - tid;
  uint64_t y = 0;
  if (e >= 0) y = h[4 * e + 3] + h[4 * e + 2] + h[4 * e + 1] + h[4 * e];
  const int sh = (e > 0 ? e : 1) - 1;
  // y * 2^sh spread over limbs j0, j0+1, j0+2
  const int j0 = sh >> 5, o = sh & 31;
  const uint64_t lo64 = y << o;
  const uint64_t top = o ? (y >> (64 - o)) : 0ull;
  uint64_t own[kLimbs], inc[kLimbs];
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    own[j] = j == j0 ? (lo64 & 0xFFFFFFFFull) : (j == j0 + 1 ? (lo64 >> 32) : (j == j0 + 2 ? top : 0ull));
    if (e < 0) own[j] = 0;
    inc[j] = own[j];
  }
  // inclusive per-limb scan in thread order (each partial sum stays below 2^43)
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t v = shfl_up64(inc[j], off);
      if (lane >= off) inc[j] += v;
    }
    if (lane == 63) s_wtot[wv][j] = inc[j];
  }
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
#pragma unroll
    for (int j = 0; j < kLimbs; ++j) inc[j] += s_wtot[w][j];
  }
  uint64_t exc[kLimbs];
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) exc[j] = inc[j] - own[j];
  const Big C = normalize(inc), E = normalize(exc);
  if (tid == 255) s_total = C;
  __syncthreads();
  if (tid == 0) {
    const uint32_t pb = __float_as_uint(top_p);
    const uint32_t pe = (pb >> 23) & 0xFFu, pm = pb & 0x7FFFFFu;
    const uint32_t mp = pe ? (pm | 0x800000u) : pm;
    const int k = 150 - (pe ? (int)pe : 1);        // p = mp * 2^-k, k >= 23 for p <= 1
    if (mp == 0 || big_zero(s_total)) {
      st.mode = 2u;                                // target 0: no hits
    } else {
      s_target = topp_target(s_total, mp, k);
      st.mode = 0u;
    }
    st.prefix = 0;
    st.mask = 0;
  }
  __syncthreads();
  if (st.mode == 0u && e >= 0 && y != 0 && big_less(E, s_target) && !big_less(C, s_target)) {
    // the boundary lies in exponent E: what the prefix still needs, in units of 2^sh
    const uint64_t need = big_shr_ceil64(big_sub(s_target, E), sh);
    uint64_t cum = 0;
    for (int b = 4 * e + 3; b >= 4 * e; --b) {
      if (cum + h[b] >= need) {
        st.rem = need - cum;
        st.prefix = (uint32_t)b << 21;
        st.mask = 2047u << 21;
        break;
      }
      cum += h[b];
    }
  }
}

// Block-wide (every thread calls it), once h holds a pass's complete weighted histogram
// and st the state before the pass: fixes the pass's digit (pass 0: the boundary
// exponent's bin, from exact multi-word sums) and narrows st; after pass 2, st.c_eq.
__device__ __forceinline__ void decide_digit(const unsigned long long* h, float top_p, int pass, ToppState& st,
                             uint64_t* s_wsum, uint64_t (*s_wtot)[kLimbs], Big& s_total, Big& s_target) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int shift = pass_shift(pass);
  const uint32_t dmask = pass_dmask(pass);
  if (pass == 0) {
    topp_first_digit(h, top_p, st, s_wtot, s_total, s_target);
    __syncthreads();
  } else {
    // every candidate shares the exponent: weights are uint64 sums of M.
    // thread t owns bins 2047-2t and 2046-2t (descending)
    const uint64_t c0 = h[kBins - 1 - 2 * tid], c1 = h[kBins - 2 - 2 * tid];
    uint64_t incl = c0 + c1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t v = shfl_up64(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    const uint64_t rem = st.rem;
    uint64_t before = 0;
    for (int w = 0; w < wv; ++w) before += s_wsum[w];
    const uint64_t excl = before + incl - (c0 + c1);
    int digit = -1;
    uint64_t above = 0;
    if (excl < rem && excl + c0 >= rem) {
      digit = kBins - 1 - 2 * tid;
      above = excl;
    } else if (excl + c0 < rem && excl + c0 + c1 >= rem) {
      digit = kBins - 2 - 2 * tid;
      above = excl + c0;
    }
    __syncthreads();
    if (digit >= 0) {
      st.rem = rem - above;
      st.prefix |= (uint32_t)digit << shift;
      st.mask |= dmask << shift;
    }
    __syncthreads();
    if (pass == 2 && tid == 0) {
      // entries equal to the boundary score all weigh M*; c of them complete the target
      const uint64_t ws = weight(__uint_as_float(st.prefix));
      st.c_eq = ws ? (int64_t)((st.rem + ws - 1) / ws) : 0;
    }
  }
}

// Adds the weights of the candidate entries of [begin, end) (positive finite scores
// whose bits match `prefix` under `mask`) to the LDS histogram h, by this pass's digit.
__device__ __forceinline__ void hist_entries(const LrfuArgs& a, int64_t begin, int64_t end, int pass,
                                             uint32_t prefix, uint32_t mask, unsigned long long* h) {
  const int shift = pass_shift(pass);
  const uint32_t dmask = pass_dmask(pass);
  for (int64_t i0 = begin; i0 < end; i0 += kThreads) {
    const int64_t i = i0 + threadIdx.x;
    const float s = i < end ? item_score(a, i) : 0.f;
    const uint64_t w = weight(s);
    const uint32_t key = __float_as_uint(s);
    hist_add(h, w != 0 && (key & mask) == prefix, (key >> shift) & dmask, w);
  }
}

__global__ __launch_bounds__(kThreads) void lrfu_hist_kernel(LrfuArgs a, int pass) {
  __shared__ unsigned long long h[kBins];
  __shared__ uint64_t s_wsum[kWaves];
  __shared__ uint64_t s_wtot[kWaves][kLimbs];
  __shared__ Big s_total, s_target;
  __shared__ int s_last;
  __shared__ ToppState st;
  const int tid = threadIdx.x;
  for (int b = tid; b < kBins; b += kThreads) h[b] = 0;
  __syncthreads();
  const uint32_t mode = pass == 0 ? 0u : a.st->mode;
  if (mode != 0) return;                      // no hits (every block reads the same word)
  const uint32_t prefix = pass == 0 ? 0u : a.st->prefix;
  const uint32_t mask = pass == 0 ? 0u : a.st->mask;

  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
  hist_entries(a, begin, end, pass, prefix, mask, h);
  __syncthreads();
  // the block's non-zero bins go into the pass's global histogram (integer atomics:
  // exact, so the order of the blocks does not matter)
  unsigned long long* gh = a.hist + (int64_t)pass * kBins;
  for (int b = tid; b < kBins; b += kThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
  // Every wave waits for its own atomics; then one thread makes the block's results
  // visible device-wide (the release writes back the whole L2, so one per block
  // suffices) and takes the ticket.
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

  // ---- last block: the pass's global weighted histogram (integer sums), then the digit
  for (int b = tid; b < kBins; b += kThreads) h[b] = __atomic_load_n(&gh[b], __ATOMIC_RELAXED);
  __syncthreads();
  if (tid == 0) st = *a.st;
  __syncthreads();
  decide_digit(h, a.top_p, pass, st, s_wsum, s_wtot, s_total, s_target);
  if (tid == 0) {
    st.ticket = 0;
    *a.st = st;
    __threadfence();
  }
}

__device__ __forceinline__ bool boundary_equal(const LrfuArgs& a, const ToppState& st, float s) {
  return st.mode == 0 && has_weight(s) && __float_as_uint(s) == st.prefix;
}

__global__ __launch_bounds__(kThreads) void lrfu_count_kernel(LrfuArgs a) {
  __shared__ uint32_t s_eq;
  if (threadIdx.x == 0) s_eq = 0;
  __syncthreads();
  const ToppState st = *a.st;
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
  uint32_t eq = 0;
  if (st.mode == 0)
    for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) eq += boundary_equal(a, st, item_score(a, i));
  if (eq) atomicAdd(&s_eq, eq);
  __syncthreads();
  if (threadIdx.x == 0) a.counts[blockIdx.x] = s_eq;
}

// Exclusive prefix of a per-thread flag over the block, in thread order.
__device__ __forceinline__ uint32_t block_scan(bool flag, uint32_t* s_wave, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(flag);
  const uint64_t below = lane == 0 ? 0ull : (bal & (~0ull >> (64 - lane)));
  if (lane == 0) s_wave[wv] = (uint32_t)__popcll(bal);
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    before += w < wv ? s_wave[w] : 0u;
    tot += s_wave[w];
  }
  __syncthreads();
  total = tot;
  return before + (uint32_t)__popcll(below);
}

// Walks entries [begin, end) in index order, given the entries equal to the boundary
// before `begin`, and writes each keep score (and hit flag).
__device__ __forceinline__ void update_entries(const LrfuArgs& a, int64_t begin, int64_t end, const ToppState& st,
                                               int64_t eq_before, uint32_t* s_wave) {
  const bool any = st.mode == 0;
  for (int64_t base = begin; base < end; base += kThreads) {
    const int64_t i = base + threadIdx.x;
    const bool valid = i < end;
    const float s = valid ? item_score(a, i) : 0.f;
    const bool eq = valid && any && boundary_equal(a, st, s);
    uint32_t eq_total;
    const uint32_t eq_rank = block_scan(eq, s_wave, eq_total);
    const bool hit = valid && any && has_weight(s) &&
                     (__float_as_uint(s) > st.prefix || (eq && eq_before + (int64_t)eq_rank < st.c_eq));
    if (valid) {
      a.keep_score[i] = a.decay * a.keep_score[i] + (hit ? s : 0.f);
      if (a.hit) a.hit[i] = (uint8_t)hit;
    }
    eq_before += eq_total;
  }
}

__global__ __launch_bounds__(kThreads) void lrfu_update_kernel(LrfuArgs a) {
  __shared__ uint32_t s_wave[kWaves];
  __shared__ int64_t s_eq_before;
  const ToppState st = *a.st;
  if (threadIdx.x == 0) {
    int64_t eqb = 0;
    for (int b = 0; b < (int)blockIdx.x; ++b) eqb += a.counts[b];
    s_eq_before = eqb;
  }
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
  update_entries(a, begin, end, st, s_eq_before, s_wave);
}

// ---- rows that fit one block (at most kMaxPerBlock entries): every step in one launch,
// the state and the three weighted histograms in LDS, no count pass (no other blocks)
// and no workspace memory touched.
__global__ __launch_bounds__(kThreads) void lrfu_one_block_kernel(LrfuArgs a) {
  __shared__ unsigned long long h[kBins];
  __shared__ uint64_t s_wsum[kWaves];
  __shared__ uint64_t s_wtot[kWaves][kLimbs];
  __shared__ Big s_total, s_target;
  __shared__ uint32_t s_wave[kWaves];
  __shared__ ToppState st;
  const int tid = threadIdx.x;
  if (tid == 0) {
    ToppState z;
    z.prefix = 0;
    z.mask = 0;
    z.mode = 0;
    z.ticket = 0;
    z.pad0 = 0;
    z.pad1 = 0;
    z.rem = 0;
    z.c_eq = 0;
    st = z;
  }
  for (int pass = 0; pass < 3; ++pass) {
    for (int b = tid; b < kBins; b += kThreads) h[b] = 0;
    __syncthreads();   // also closes the previous pass's reads of h and its update of st
    if (st.mode != 0) break;   // no hits (uniform)
    hist_entries(a, 0, a.n, pass, st.prefix, st.mask, h);
    __syncthreads();
    decide_digit(h, a.top_p, pass, st, s_wsum, s_wtot, s_total, s_target);
  }
  __syncthreads();
  update_entries(a, 0, a.n, st, 0, s_wave);
}

}  // namespace

int lrfu_blocks(int64_t n) {
  if (n <= kMaxPerBlock) return 1;
  int64_t b = (n + kPerBlock - 1) / kPerBlock;
  if (b > kMaxBlocks) b = kMaxBlocks;
  return (int)b;
}

size_t lrfu_workspace_bytes(int64_t n) {
  const int nb = lrfu_blocks(n);
  return 256 + (size_t)3 * kBins * sizeof(unsigned long long) + (size_t)nb * sizeof(int64_t);
}

hipError_t launch_lrfu(const LrfuArgs& a, hipStream_t s) {
  if (trace_on())
    trace_launch(a.n_blocks == 1 ? "lrfu one block (3 hist passes, update) grid=%d block=%d  entries=%lld top_p=%g"
                                 : "lrfu init+3 hist+count+update grid=%d block=%d  entries=%lld top_p=%g",
                 a.n_blocks, kThreads, (long long)a.n, (double)a.top_p);
  if (a.n_blocks == 1) {
    // the whole row fits one block: one launch instead of six
    hipLaunchKernelGGL(lrfu_one_block_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(lrfu_init_kernel, dim3(1), dim3(kThreads), 0, s, a.st, a.hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.n_blocks), block(kThreads);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(lrfu_hist_kernel, grid, block, 0, s, a, pass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lrfu_count_kernel, grid, block, 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(lrfu_update_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
