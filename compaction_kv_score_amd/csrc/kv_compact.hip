// Stable in-order gather compaction with exact re-rotation of the kept keys.
//
// ActKV (Sec. 3.3, 7.2) makes compaction the second system bottleneck: evicted tokens
// leave holes across pages that must be closed.  PACE (Sec. 3.2) renumbers the kept row
// in logical order (order-preserving, gap-collapsing) and re-rotates every kept key
// from its old to its new position; Proposition 1 states that rotating a cached key by
// the position difference gives exactly the key the model would have cached there.
//
// One workgroup moves one kept token: for every layer and KV head it reads the token's
// K and V rows (16-byte loads; a thread owns the 8-dim chunk c and its RoPE partner
// c + 64 of one head, i.e. dims 8c..8c+7 and 64+8c..64+8c+7) and writes them to the
// destination slot of its rank.  V is copied bit for bit.  K is copied bit for bit when
// the position does not change; otherwise each split-half pair (x_i, x_{i+64}) is
// rotated by delta * theta_i, theta_i = base^(-2i/128), with the 64 cos/sin values of
// the token computed once in float64 into LDS, the rotation done in float64 from the
// exact bf16 inputs, and one round-to-nearest-even to bf16.
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kCompactThreads = 256;

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// float64 -> bf16 bits, round to nearest, ties to even, from the definition: keep the
// top 8 significant bits.  Normal range: add half an ulp (plus the tie-to-even bit) at
// bit 45 of the float64 pattern and truncate; the result is exactly representable in
// float32, whose top half is the bf16 pattern.  Below 2^-126 the bf16 spacing is fixed
// at 2^-133, so scale by 2^133 (exact) and round to an integer.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  const double av = fabs(v);
  if (!(av >= 0x1p-126)) {
    if (v != v) return 0x7FC0u | ((uint32_t)(__double_as_longlong(v) >> 48) & 0x8000u);
    const double r = rint(v * 0x1p133) * 0x1p-133;
    return __float_as_uint((float)r) >> 16;
  }
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u += 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~0x1FFFFFFFFFFFull;
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}

__device__ __forceinline__ int64_t source_token(const CompactArgs& a, int64_t r) {
  if (a.keep) return a.keep[r];
  return r >= a.split ? r + a.shift : r;
}

__device__ __forceinline__ void rotate_chunk(uint4& lo, uint4& hi, const double2* cs) {
  uint32_t xl[4] = {lo.x, lo.y, lo.z, lo.w};
  uint32_t yl[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t xo = 0, yo = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t xb = (xl[q] >> (16 * half)) & 0xFFFFu;
      const uint32_t yb = (yl[q] >> (16 * half)) & 0xFFFFu;
      const double x = bf16_to_f64(xb);
      const double y = bf16_to_f64(yb);
      const double2 t = cs[2 * q + half];
      const double xr = x * t.x - y * t.y;
      const double yr = x * t.y + y * t.x;
      xo |= f64_to_bf16_rne(xr) << (16 * half);
      yo |= f64_to_bf16_rne(yr) << (16 * half);
    }
    xl[q] = xo;
    yl[q] = yo;
  }
  lo = make_uint4(xl[0], xl[1], xl[2], xl[3]);
  hi = make_uint4(yl[0], yl[1], yl[2], yl[3]);
}

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactArgs a) {
  __shared__ double2 cs[64];
  const int tid = threadIdx.x;
  const int64_t r = a.rank0 + blockIdx.x;
  if (r >= a.rank1) return;
  if (a.n_keep && r >= *a.n_keep) return;
  const int64_t j = source_token(a, r);
  const int32_t op = a.old_pos[j];
  const int32_t np = a.renumber_base >= 0 ? a.renumber_base + (int32_t)r : op;
  const int64_t delta = (int64_t)np - (int64_t)op;
  const bool in_place = a.keep == nullptr && j == r && a.src_k == a.dst_k;
  if (in_place && delta == 0) return;  // already where it belongs

  if (delta != 0) {
    if (tid < 64) {
      const double inv = exp(-(2.0 * tid / kHeadDim) * a.log_theta);
      double s, c;
      sincos((double)delta * inv, &s, &c);
      cs[tid] = make_double2(c, s);
    }
    __syncthreads();
  }

  const int slot_stride = a.n_kv_heads * kHeadDim;
  const int64_t src_off = token_offset(j, a.src_page_shift, a.src_page_stride, a.src_bt, slot_stride);
  const int64_t dst_off = token_offset(r, a.dst_page_shift, a.dst_page_stride, a.dst_bt, slot_stride);
  const int per_layer = a.n_kv_heads * 8;
  const int items = a.n_layers * per_layer;
#pragma unroll 2
  for (int e = tid; e < items; e += kCompactThreads) {
    const int layer = e / per_layer;
    const int rem = e - layer * per_layer;
    const int h = rem >> 3;
    const int cidx = rem & 7;
    const int64_t so = (int64_t)layer * a.src_layer_stride + src_off + h * kHeadDim + cidx * 8;
    const int64_t d_o = (int64_t)layer * a.dst_layer_stride + dst_off + h * kHeadDim + cidx * 8;
    uint4 klo = *(const uint4*)(a.src_k + so);
    uint4 khi = *(const uint4*)(a.src_k + so + 64);
    uint4 vlo, vhi;
    if (!in_place) {
      vlo = *(const uint4*)(a.src_v + so);
      vhi = *(const uint4*)(a.src_v + so + 64);
    }
    if (delta != 0) rotate_chunk(klo, khi, &cs[cidx * 8]);
    *(uint4*)(a.dst_k + d_o) = klo;
    *(uint4*)(a.dst_k + d_o + 64) = khi;
    if (!in_place) {
      *(uint4*)(a.dst_v + d_o) = vlo;
      *(uint4*)(a.dst_v + d_o + 64) = vhi;
    }
  }
}

// New positions and per-token metadata, one thread per rank (coalesced over ranks).
__global__ __launch_bounds__(256) void gather_meta_kernel(CompactArgs a) {
  const int64_t r = a.rank0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= a.rank1) return;
  if (a.n_keep && r >= *a.n_keep) return;
  const int64_t j = source_token(a, r);
  if (a.new_pos) a.new_pos[r] = a.renumber_base >= 0 ? a.renumber_base + (int32_t)r : a.old_pos[j];
  for (int m = 0; m < a.meta.n; ++m) {
    switch (a.meta.elem_bytes[m]) {
      case 1:
        ((uint8_t*)a.meta.dst[m])[r] = ((const uint8_t*)a.meta.src[m])[j];
        break;
      case 2:
        ((uint16_t*)a.meta.dst[m])[r] = ((const uint16_t*)a.meta.src[m])[j];
        break;
      case 4:
        ((uint32_t*)a.meta.dst[m])[r] = ((const uint32_t*)a.meta.src[m])[j];
        break;
      default:
        ((uint64_t*)a.meta.dst[m])[r] = ((const uint64_t*)a.meta.src[m])[j];
        break;
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const int64_t n = a.rank1 - a.rank0;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)n), dim3(kCompactThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_meta(const CompactArgs& a, hipStream_t s) {
  const int64_t n = a.rank1 - a.rank0;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_meta_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
