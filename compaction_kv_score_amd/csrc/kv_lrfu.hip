// ActKV's attention-aware LRFU keep scores (ActKV Sec. 5.1, Algorithm 1) on gfx950.
//
//   KS <- decay * KS + AttnScore   for hits,   KS <- decay * KS   for misses,
// where an entry is a hit when its score lies in the top-p set: the smallest prefix of
// the entries in the total order (score descending, index ascending) whose weight
// reaches ceil(p * W).  Weights are fixed-point, w = floor(s * 2^shift) for finite s > 0
// (0 otherwise), with shift chosen from the largest score and the entry count so that
// the total W stays below 2^52; every sum is then exact integer arithmetic and the hit
// set does not depend on the order of the additions.
//
// Steps (no host synchronisation):
//   1. the largest score (integer atomic max of its bits);
//   2. three weighted radix passes over the 11-, 11- and 10-bit digits of the score bits:
//      per-block LDS histograms of weight sums (64-bit integer atomics), merged by the
//      last block in block order, which fixes the digit where the weight counted from
//      the top reaches what is still missing of the target.  Afterwards T is the
//      boundary score and c the number of entries equal to T (lowest indices first)
//      that complete the target;
//   3. a count pass (entries equal to T per block) and an update pass that walks the
//      entries in index order, decides hits and writes KS (and the hit mask).
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 64;
constexpr int kBins = 2048;
// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt not waited for
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

__device__ __forceinline__ bool has_weight(float s) { return s > 0.f && s <= 3.402823466e38f; }

__device__ __forceinline__ int weight_shift(uint32_t max_bits, int64_t n) {
  int e;
  frexpf(__uint_as_float(max_bits), &e);          // max < 2^e
  const int lg = n > 1 ? 64 - __clzll((unsigned long long)(n - 1)) : 0;  // ceil(log2 n)
  return 52 - lg - e;
}

__device__ __forceinline__ uint64_t weight(float s, int shift) {
  return has_weight(s) ? (uint64_t)floor(ldexp((double)s, shift)) : 0ull;
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

__global__ __launch_bounds__(64) void lrfu_init_kernel(ToppState* st) {
  if (threadIdx.x == 0) {
    ToppState z;
    z.prefix = 0;
    z.mask = 0;
    z.mode = 0;
    z.ticket = 0;
    z.max_bits = 0;
    z.pad = 0;
    z.rem = 0;
    z.total = 0;
    z.c_eq = 0;
    *st = z;
  }
}

__device__ __forceinline__ float item_score(const LrfuArgs& a, int64_t i) { return a.score[i] * a.scale; }

__global__ __launch_bounds__(kThreads) void lrfu_max_kernel(LrfuArgs a) {
  __shared__ uint32_t s_max;
  if (threadIdx.x == 0) s_max = 0;
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
  uint32_t m = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
    const float s = item_score(a, i);
    if (has_weight(s)) m = max(m, __float_as_uint(s));   // positive floats order as integers
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(&s_max, m);
  __syncthreads();
  if (threadIdx.x == 0 && s_max) atomicMax(&a.st->max_bits, s_max);
}

__global__ __launch_bounds__(kThreads) void lrfu_hist_kernel(LrfuArgs a, int pass) {
  __shared__ unsigned long long h[kBins];
  __shared__ uint64_t s_wsum[kWaves];
  __shared__ int s_last;
  __shared__ ToppState st;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int b = tid; b < kBins; b += kThreads) h[b] = 0;
  __syncthreads();
  const uint32_t max_bits = a.st->max_bits;
  if (max_bits == 0) return;                  // no entry carries weight: no hits
  const uint32_t mode = pass == 0 ? 0u : a.st->mode;
  if (mode != 0) return;
  const uint32_t prefix = pass == 0 ? 0u : a.st->prefix;
  const uint32_t mask = pass == 0 ? 0u : a.st->mask;
  const int shift = pass_shift(pass);
  const uint32_t dmask = pass_dmask(pass);
  const int wsh = weight_shift(max_bits, a.n);

  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
  for (int64_t i0 = begin; i0 < end; i0 += kThreads) {
    const int64_t i = i0 + tid;
    const float s = i < end ? item_score(a, i) : 0.f;
    const uint64_t w = weight(s, wsh);
    const uint32_t key = __float_as_uint(s);
    hist_add(h, w != 0 && (key & mask) == prefix, (key >> shift) & dmask, w);
  }
  __syncthreads();
  for (int b = tid; b < kBins; b += kThreads) a.hist[(int64_t)blockIdx.x * kBins + b] = h[b];
  // Every wave waits for its own stores; then one thread makes the block's histogram
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

  // ---- last block: global weighted histogram (blocks in order), then the digit
  const int nb = (int)gridDim.x;
  for (int b = tid; b < kBins; b += kThreads) {
    unsigned long long tot = 0;
    for (int blk = 0; blk < nb; ++blk)
      tot += __atomic_load_n(&a.hist[(int64_t)blk * kBins + b], __ATOMIC_RELAXED);
    h[b] = tot;
  }
  __syncthreads();
  if (tid == 0) st = *a.st;
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
  if (pass == 0 && tid == 0) {
    uint64_t total = 0;
    for (int w = 0; w < kWaves; ++w) total += s_wsum[w];
    const double target = ceil((double)a.top_p * (double)total);
    st.total = total;
    st.rem = target > 0.0 ? (uint64_t)target : 0ull;
    st.mode = st.rem == 0 ? 2u : 0u;
    st.prefix = 0;
    st.mask = 0;
  }
  __syncthreads();
  if (st.mode == 0) {
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
    if (digit >= 0) {
      st.rem = rem - above;
      st.prefix |= (uint32_t)digit << shift;
      st.mask |= dmask << shift;
    }
    __syncthreads();
    if (pass == 2 && tid == 0) {
      // entries equal to the boundary score all weigh w*; c of them complete the target
      const uint64_t ws = weight(__uint_as_float(st.prefix), wsh);
      st.c_eq = ws ? (int64_t)((st.rem + ws - 1) / ws) : 0;
    }
  }
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
  if (st.max_bits != 0)
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

__global__ __launch_bounds__(kThreads) void lrfu_update_kernel(LrfuArgs a) {
  __shared__ uint32_t s_wave[kWaves];
  __shared__ int64_t s_eq_before;
  const ToppState st = *a.st;
  const bool any = st.max_bits != 0 && st.mode == 0;
  if (threadIdx.x == 0) {
    int64_t eqb = 0;
    for (int b = 0; b < (int)blockIdx.x; ++b) eqb += a.counts[b];
    s_eq_before = eqb;
  }
  __syncthreads();
  int64_t eq_before = s_eq_before;
  const int64_t begin = (int64_t)blockIdx.x * a.per_block;
  const int64_t end = begin + a.per_block < a.n ? begin + a.per_block : a.n;
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

}  // namespace

int lrfu_blocks(int64_t n) {
  int64_t b = (n + 4095) / 4096;
  if (b < 1) b = 1;
  if (b > kMaxBlocks) b = kMaxBlocks;
  return (int)b;
}

size_t lrfu_workspace_bytes(int64_t n) {
  const int nb = lrfu_blocks(n);
  return 256 + (size_t)nb * kBins * sizeof(unsigned long long) + (size_t)nb * sizeof(int64_t);
}

hipError_t launch_lrfu(const LrfuArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lrfu_init_kernel, dim3(1), dim3(64), 0, s, a.st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.n_blocks), block(kThreads);
  hipLaunchKernelGGL(lrfu_max_kernel, grid, block, 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
