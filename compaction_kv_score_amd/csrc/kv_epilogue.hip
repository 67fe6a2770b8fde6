// Per-token policy epilogue of kv_score.
//
// Reduces the per-(layer, KV head) attention-mass partials of one token in a fixed
// order (float64 accumulation), then applies the retention policy:
//   MemDecay (MemDecay, Method): Abar = mass / (L*Hq*W), the mean of the weights over
//     layers, query heads and window queries; a <- rho*a + (1-rho)*Abar; the decay clock
//     resets when Abar > tau and otherwise advances by dt_steps;
//     s = b_r * exp(-lambda_r * clock) + alpha * a.
//   H2O (PACE Sec. 2, heavy hitters): acc <- acc + mass; s = acc.
// plus the foresight bonus of the token's span, one value per span from the caller's
// planner (PACE Sec. 3.1 and 7), and the pinning rules (MemDecay pinned regions, PACE
// Table 1 sinks and recent window).  In page mode a page's score is the mean over the
// tokens it holds (MemDecay's S_p) and a page is pinned when any token is.
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kEpiThreads = 256;   // tokens per block
constexpr int kEpiSplit = 4;       // threads sharing one token's partials

__global__ __launch_bounds__(kEpiThreads * kEpiSplit) void epilogue_kernel(EpilogueArgs a) {
  __shared__ float s_sum[kEpiThreads];
  __shared__ int s_cnt[kEpiThreads];
  __shared__ int s_pin[kEpiThreads];
  __shared__ double s_part[kEpiSplit][kEpiThreads];
  const int tid = threadIdx.x % kEpiThreads;
  const int quarter = threadIdx.x / kEpiThreads;
  const int64_t N = a.n_tokens;
  const int64_t i = (int64_t)blockIdx.x * kEpiThreads + tid;
  const bool valid = i < N;

  // Fixed-order float64 sum of the partials: thread `quarter` adds a contiguous quarter
  // of them in order (loads issued 8 at a time so that enough are in flight), and the
  // four quarter sums are added in quarter order.
  {
    const int per = (a.n_parts + kEpiSplit - 1) / kEpiSplit;
    const int p0 = quarter * per;
    const int p1 = p0 + per < a.n_parts ? p0 + per : a.n_parts;
    double qsum = 0.0;
    if (valid) {
      const float* mp = a.mass_part + i;
      int p = p0;
      for (; p + 8 <= p1; p += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = mp[(int64_t)(p + k) * N];
#pragma unroll
        for (int k = 0; k < 8; ++k) qsum += (double)v[k];
      }
      for (; p < p1; ++p) qsum += (double)mp[(int64_t)p * N];
    }
    s_part[quarter][tid] = qsum;
  }
  __syncthreads();

  float score = 0.f;
  int pinned = 0;
  bool bad_region = false;
  if (valid && quarter == 0) {
    double msum = s_part[0][tid];
#pragma unroll
    for (int q = 1; q < kEpiSplit; ++q) msum += s_part[q][tid];
    const float mass = (float)msum;
    if (a.mass) a.mass[i] = mass;

    float bonus = 0.f;
    if (a.span_id) {
      const int sid = a.span_id[i];
      if (sid >= 0 && sid < a.n_spans) bonus = a.span_bonus[sid];
    }
    // a label outside the region table names no region (reported through the status)
    int r = 0;
    if (a.region) {
      r = a.region[i];
      if (r >= a.n_regions) {
        bad_region = true;
        r = 0;
      }
    }
    if (a.policy == KV_POLICY_MEMDECAY) {
      const float abar = (float)(msum * a.mass_norm);
      const float ew = a.rho * a.ewma[i] + (1.0f - a.rho) * abar;
      const int32_t clk = abar > a.tau ? 0 : a.clock[i] + a.dt_steps;
      a.ewma[i] = ew;
      a.clock[i] = clk;
      const float b = a.base_prio && !bad_region ? a.base_prio[r] : 0.f;
      const float lam = a.decay_rate && !bad_region ? a.decay_rate[r] : 0.f;
      score = b * expf(-lam * (float)clk) + a.alpha * ew + bonus;
    } else {
      const float acc = a.accum[i] + mass;
      a.accum[i] = acc;
      score = acc + bonus;
    }
    if (a.token_score) a.token_score[i] = score;
    pinned = (i < a.n_sink) || (i >= N - a.n_recent) ||
             (a.region && !bad_region && ((a.pinned_regions >> r) & 1u)) ||
             (a.token_pinned && a.token_pinned[i] != 0);
  }
  if (a.status && __builtin_amdgcn_ballot_w64(bad_region) != 0 && (tid & 63) == 0)
    atomicOr(a.status, KV_STATUS_BAD_REGION);

  if (a.item_shift == 0) {
    if (valid && quarter == 0) {
      a.item_score[i] = score;
      a.item_pinned[i] = (uint8_t)pinned;
    }
    return;
  }
  // page mode: pairwise reduction inside each aligned segment of item_tokens threads
  // (the first kEpiThreads threads; every thread reaches every barrier)
  if (quarter == 0) {
    s_sum[tid] = valid ? score : 0.f;
    s_cnt[tid] = valid ? 1 : 0;
    s_pin[tid] = pinned;
  }
  __syncthreads();
  const int it = 1 << a.item_shift;
  for (int stride = 1; stride < it; stride <<= 1) {
    if (quarter == 0 && (tid & (2 * stride - 1)) == 0) {
      s_sum[tid] += s_sum[tid + stride];
      s_cnt[tid] += s_cnt[tid + stride];
      s_pin[tid] |= s_pin[tid + stride];
    }
    __syncthreads();
  }
  if (quarter == 0 && (tid & (it - 1)) == 0 && s_cnt[tid] > 0) {
    const int64_t page = i >> a.item_shift;
    a.item_score[page] = s_sum[tid] / (float)s_cnt[tid];
    a.item_pinned[page] = (uint8_t)(s_pin[tid] != 0);
  }
}

}  // namespace

hipError_t launch_epilogue(const EpilogueArgs& a, hipStream_t s) {
  const int64_t blocks = (a.n_tokens + kEpiThreads - 1) / kEpiThreads;
  if (trace_on())
    trace_launch("epilogue grid=%lld block=%d  tokens=%lld partials=%d policy=%s items_of=%d", (long long)blocks,
                 kEpiThreads * kEpiSplit, (long long)a.n_tokens, a.n_parts,
                 a.policy == KV_POLICY_MEMDECAY ? "memdecay" : "h2o", 1 << a.item_shift);
  hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)blocks), dim3(kEpiThreads * kEpiSplit), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
