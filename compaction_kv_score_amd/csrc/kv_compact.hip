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
// rotated by delta * theta_i, with theta_i from the caller's frequency table (plain
// base^(-2i/128) or a static scaling, PACE Sec. 3.5), the 64 cos/sin values of the
// token computed once in float64 into LDS, the rotation done in float64 from the exact
// bf16 inputs, and one round-to-nearest-even to bf16.
//
// With a reference store (PACE Sec. 3.2, non-compounding re-rotation) the workgroup
// first checks the source slot's entry: the stored key re-rotated to the token's current
// position and rounded must equal the cached key.  A valid entry is the rotation source
// (and moves to the destination slot); otherwise a key whose position changes is stored
// with its current position before it is rotated.
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kCompactThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: the kept rows are read once, and the hint keeps
// them from displacing other cached data.
__device__ __forceinline__ uint4 load_once(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte store marked non-temporal: streams to memory without allocating in the caches.
__device__ __forceinline__ void store_once(uint16_t* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)p);
}

template <bool kNt>
__device__ __forceinline__ void store16(uint16_t* p, const uint4& v) {
  if constexpr (kNt) store_once(p, v);
  else *(uint4*)p = v;
}

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

// Value equality of two bf16 patterns: +0 equals -0 and NaN equals nothing.
__device__ __forceinline__ bool bf16_same(uint32_t x, uint32_t y) {
  const uint32_t mx = x & 0x7FFFu, my = y & 0x7FFFu;
  if (mx > 0x7F80u || my > 0x7F80u) return false;
  return x == y || (mx == 0 && my == 0);
}

__device__ __forceinline__ bool chunk_same(const uint4& p, const uint4& q) {
  const uint32_t pv[4] = {p.x, p.y, p.z, p.w};
  const uint32_t qv[4] = {q.x, q.y, q.z, q.w};
  bool same = true;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    same = same && bf16_same(pv[w] & 0xFFFFu, qv[w] & 0xFFFFu) && bf16_same(pv[w] >> 16, qv[w] >> 16);
  return same;
}

// cos/sin of delta * theta_i for the 64 pairs, in float64.
__device__ __forceinline__ void fill_rotation(double2* cs, const CompactArgs& a, int64_t delta, int tid) {
  if (tid < kHeadDim / 2) {
    double s, c;
    sincos((double)delta * a.inv_freq[tid], &s, &c);
    cs[tid] = make_double2(c, s);
  }
}

// Per-token metadata of rank r taken from source token j (element sizes 1, 2, 4 or 8).
__device__ __forceinline__ void gather_meta_row(const MetaSet& m, int64_t j, int64_t r) {
  for (int i = 0; i < m.n; ++i) {
    switch (m.elem_bytes[i]) {
      case 1:
        ((uint8_t*)m.dst[i])[r] = ((const uint8_t*)m.src[i])[j];
        break;
      case 2:
        ((uint16_t*)m.dst[i])[r] = ((const uint16_t*)m.src[i])[j];
        break;
      case 4:
        ((uint32_t*)m.dst[i])[r] = ((const uint32_t*)m.src[i])[j];
        break;
      default:
        ((uint64_t*)m.dst[i])[r] = ((const uint64_t*)m.src[i])[j];
        break;
    }
  }
}

template <bool kStore, bool kNt>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactArgs a) {
  __shared__ double2 cs[64];
  __shared__ double2 cs_chk[kStore ? 64 : 1];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int64_t r = a.rank0 + blockIdx.x / a.parts;
  const int part = (int)(blockIdx.x % a.parts);
  if (r >= a.rank1) return;
  if (a.n_keep && r >= *a.n_keep) return;
  const int64_t j = source_token(a, r);
  if (j < 0 || j >= a.src_tokens) return;   // malformed keep entry: nothing is read or written
  const int32_t op = a.old_pos[j];
  const int32_t np = a.renumber_base >= 0 ? a.renumber_base + (int32_t)r : op;

  const int slot_stride = a.n_kv_heads * kHeadDim;
  const int64_t src_off = token_offset(j, a.src_page_shift, a.src_page_stride, a.src_bt, slot_stride);
  const int64_t dst_off = token_offset(r, a.dst_page_shift, a.dst_page_stride, a.dst_bt, slot_stride);
  // the token's key and value already sit in its destination slot (the in-place forms):
  // V is not copied, and K is rewritten only when it is re-rotated
  const bool in_place = a.src_k == a.dst_k && src_off == dst_off;
  if (in_place && np == op && a.rows_in_place) return;  // nothing to write, store entry included
  if (a.remap_only && !in_place) {                      // not a whole-page keep entry: left alone
    if (tid == 0 && part == 0 && a.status) atomicOr(a.status, KV_STATUS_NOT_WHOLE_PAGES);
    return;
  }
  const int per_layer = a.n_kv_heads * 8;
  const int items = a.n_layers * per_layer;

  int32_t rp = KV_REF_NONE;
  bool use_ref = false;
  if (kStore) {
    rp = a.ref_src_pos[j];
    if (rp != KV_REF_NONE) {
      // check the entry against the cached key at its current position
      fill_rotation(cs_chk, a, (int64_t)op - rp, tid);
      if (tid == 0) s_bad = 0;
      __syncthreads();
      bool bad = false;
      for (int e = tid; e < items; e += kCompactThreads) {
        const int layer = e / per_layer;
        const int rem = e - layer * per_layer;
        const int64_t col = (rem >> 3) * kHeadDim + (rem & 7) * 8;
        const int64_t so = (int64_t)layer * a.src_layer_stride + src_off + col;
        const int64_t ro = (int64_t)layer * a.ref_src_layer_stride + j * slot_stride + col;
        const uint4 klo = *(const uint4*)(a.src_k + so);
        const uint4 khi = *(const uint4*)(a.src_k + so + 64);
        uint4 rlo = *(const uint4*)(a.ref_src_k + ro);
        uint4 rhi = *(const uint4*)(a.ref_src_k + ro + 64);
        rotate_chunk(rlo, rhi, &cs_chk[(rem & 7) * 8]);
        bad = bad || !chunk_same(rlo, klo) || !chunk_same(rhi, khi);
      }
      if (bad) s_bad = 1;
      __syncthreads();
      use_ref = s_bad == 0;
    }
  }
  const int64_t delta = use_ref ? (int64_t)np - rp : (int64_t)np - op;
  const bool seed = kStore && !use_ref && np != op;
  const bool move_entry = kStore && use_ref && !(a.ref_dst_k == a.ref_src_k && j == r);
  if (delta != 0) {
    fill_rotation(cs, a, delta, tid);
    __syncthreads();
  }

  // this workgroup's share of the (layer, head, chunk pair) items; none when the token
  // stays in its slot unrotated (only its position and metadata are written below)
  const bool touch = !(in_place && delta == 0 && !seed && !move_entry);
  const int e0 = touch ? (int)((int64_t)part * items / a.parts) : 0;
  const int e1 = touch ? (int)((int64_t)(part + 1) * items / a.parts) : 0;
#pragma unroll 2
  for (int e = e0 + tid; e < e1; e += kCompactThreads) {
    const int layer = e / per_layer;
    const int rem = e - layer * per_layer;
    const int64_t col = (rem >> 3) * kHeadDim + (rem & 7) * 8;
    const int64_t so = (int64_t)layer * a.src_layer_stride + src_off + col;
    const int64_t d_o = (int64_t)layer * a.dst_layer_stride + dst_off + col;
    uint4 klo, khi;
    if (kStore && use_ref) {
      const int64_t ro = (int64_t)layer * a.ref_src_layer_stride + j * slot_stride + col;
      klo = *(const uint4*)(a.ref_src_k + ro);
      khi = *(const uint4*)(a.ref_src_k + ro + 64);
    } else {
      klo = load_once(a.src_k + so);
      khi = load_once(a.src_k + so + 64);
    }
    if (kStore && (seed || move_entry)) {
      const int64_t rd = (int64_t)layer * a.ref_dst_layer_stride + r * slot_stride + col;
      *(uint4*)(a.ref_dst_k + rd) = klo;
      *(uint4*)(a.ref_dst_k + rd + 64) = khi;
    }
    uint4 vlo, vhi;
    if (!in_place) {
      vlo = load_once(a.src_v + so);
      vhi = load_once(a.src_v + so + 64);
    }
    if (delta != 0) rotate_chunk(klo, khi, &cs[(rem & 7) * 8]);
    store16<kNt>(a.dst_k + d_o, klo);
    store16<kNt>(a.dst_k + d_o + 64, khi);
    if (!in_place) {
      store16<kNt>(a.dst_v + d_o, vlo);
      store16<kNt>(a.dst_v + d_o + 64, vhi);
    }
  }
  // The rank's new position, metadata and store position, written by its first
  // workgroup once every wave has read the old ones (the in-place forms pass the same
  // arrays as source and destination; a launch whose ranks read positions that it also
  // writes runs one workgroup per rank).
  __syncthreads();
  if (tid == 0 && part == 0) {
    if (a.new_pos) a.new_pos[r] = np;
    gather_meta_row(a.meta, j, r);
    if (kStore) a.ref_dst_pos[r] = use_ref ? rp : (seed ? op : KV_REF_NONE);
  }
}

__global__ __launch_bounds__(256) void remap_table_kernel(const int32_t* bt, int32_t* bt_out, int32_t* freed,
                                                          int64_t keep_pages, int64_t prefix_pages,
                                                          int64_t evict_pages) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < keep_pages) bt_out[p] = bt[p < prefix_pages ? p : p + evict_pages];
  if (freed && p < evict_pages) freed[p] = bt[prefix_pages + p];
}

__global__ __launch_bounds__(256) void remap_pages_kernel(const int32_t* bt, int32_t* bt_out, const int32_t* keep,
                                                          const int64_t* n_keep, int64_t max_keep, int page_shift,
                                                          int64_t n_pages_src, uint32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i == 0 && status) *status = 0u;                  // the compaction, next on the stream, sets bits
  int64_t n = n_keep ? *n_keep : max_keep;
  n = n < max_keep ? n : max_keep;
  const int64_t page = (int64_t)1 << page_shift;
  if (i * page >= n) return;
  const int64_t first = keep[i * page];
  if (first >= 0 && (first >> page_shift) < n_pages_src) bt_out[i] = bt[first >> page_shift];
}

// Positions and metadata of ranks [0, n) whose tokens keep their slot and their position
// (a remap without renumbering): one thread per rank, nothing else is touched.
__global__ __launch_bounds__(256) void remap_rows_kernel(CompactArgs a, int64_t n) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= n) return;
  const int64_t j = source_token(a, r);
  a.new_pos[r] = a.old_pos[j];
  gather_meta_row(a.meta, j, r);
}

__global__ __launch_bounds__(256) void ref_invalidate_kernel(int32_t* pos, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) pos[i] = KV_REF_NONE;
}

// Number of leading entries of a monotone predicate over [0, n) (true, then false),
// found by the whole workgroup with 256-way splits: a handful of rounds for any n.
template <class Pred>
__device__ int64_t block_count_true(int64_t n, Pred pred) {
  int64_t lo = 0, hi = n;                 // the count lies in [lo, hi]
  while (hi > lo) {
    const int64_t step = (hi - lo + kCompactThreads - 1) / kCompactThreads;
    const int64_t p = lo + (int64_t)(threadIdx.x + 1) * step - 1;
    const int m = __syncthreads_count(p < hi && pred(p));
    const int64_t nlo = lo + (int64_t)m * step;
    const int64_t nhi = lo + (int64_t)(m + 1) * step - 1;
    lo = nlo;
    hi = nhi < hi ? nhi : hi;
  }
  return lo;
}

// ActKV Sec. 7.2 / Algorithm 4: the kept entries outside the target region move into
// the region's free slots, source d to destination d in ascending order.  Workgroup d
// finds its pair by block-wide searches over the ascending keep list: the d-th source
// is keep[d] or keep[d + k_in] (k_in kept entries lie inside the region), the d-th free
// slot is start + d + c with c the kept entries inside whose own free-slot count
// keep[r] - start - (r - r_in) does not exceed d.  Sources and destinations are
// disjoint, so every copy runs at once and nothing is staged.
__global__ __launch_bounds__(kCompactThreads) void tail_compact_kernel(TailArgs a) {
  const int tid = threadIdx.x;
  int64_t n_keep = a.n_keep ? *a.n_keep : a.max_keep;
  n_keep = n_keep < a.max_keep ? n_keep : a.max_keep;
  n_keep = n_keep < 0 ? 0 : n_keep;
  const int64_t start = a.start, end = a.start + a.budget;
  const int32_t* keep = a.keep;
  const int64_t r_in = block_count_true(n_keep, [&](int64_t i) { return keep[i] < start; });
  const int64_t r_out = block_count_true(n_keep, [&](int64_t i) { return keep[i] < end; });
  const int64_t k_in = r_out - r_in;
  const int64_t n_src = n_keep - k_in, holes = a.budget - k_in;
  const int64_t n_pairs = n_src < holes ? n_src : holes;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = n_src > holes ? KV_STATUS_KEEP_OVERFLOW : 0u;
  const int64_t d = blockIdx.x;
  if (d >= n_pairs) return;
  const int64_t src = keep[d < r_in ? d : d + k_in];
  if (src < 0 || src >= a.n_tokens) return;  // malformed keep entry: nothing is moved
  const int64_t c = block_count_true(k_in, [&](int64_t i) { return keep[r_in + i] - start - i <= d; });
  const int64_t dst = start + d + c;

  const int slot_stride = a.n_kv_heads * kHeadDim;
  const int64_t so = token_offset(src, a.page_shift, a.page_stride, a.bt, slot_stride);
  const int64_t dof = token_offset(dst, a.page_shift, a.page_stride, a.bt, slot_stride);
  const int per_layer = slot_stride / 8;            // 16-byte chunks per layer
  const int items = a.n_layers * per_layer;
  for (int e = tid; e < items; e += kCompactThreads) {
    const int layer = e / per_layer;
    const int64_t col = (int64_t)(e - layer * per_layer) * 8;
    const int64_t lo = (int64_t)layer * a.layer_stride;
    const uint4 kk = load_once(a.k + lo + so + col);
    const uint4 vv = load_once(a.v + lo + so + col);
    *(uint4*)(a.k + lo + dof + col) = kk;
    *(uint4*)(a.v + lo + dof + col) = vv;
  }
  if (tid == 0) {
    for (int m = 0; m < a.meta.n; ++m) {
      switch (a.meta.elem_bytes[m]) {
        case 1: ((uint8_t*)a.meta.dst[m])[dst] = ((const uint8_t*)a.meta.src[m])[src]; break;
        case 2: ((uint16_t*)a.meta.dst[m])[dst] = ((const uint16_t*)a.meta.src[m])[src]; break;
        case 4: ((uint32_t*)a.meta.dst[m])[dst] = ((const uint32_t*)a.meta.src[m])[src]; break;
        default: ((uint64_t*)a.meta.dst[m])[dst] = ((const uint64_t*)a.meta.src[m])[src]; break;
      }
    }
  }
}

// Rows a compaction drops (PACE Sec. 3.4 offloads them at every compaction): workgroup
// e - first copies the e-th token not in the keep list, t = e + c with c the kept tokens
// whose own count of dropped tokens before them (keep[i] - i) does not exceed e.
__global__ __launch_bounds__(kCompactThreads) void gather_evicted_kernel(EvictArgs a) {
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x / a.parts;
  const int part = (int)(blockIdx.x % a.parts);
  const int64_t e = a.first + r;
  const int32_t* keep = a.keep;
  const int64_t c = block_count_true(a.n_keep, [&](int64_t i) { return keep[i] - i <= e; });
  const int64_t t = e + c;
  // a keep list that is not strictly ascending inside [0, N) can point past the row:
  // such a rank is skipped (nothing read or written), as the other copies skip theirs
  if (t < 0 || t >= a.src_tokens) return;
  const int slot_stride = a.n_kv_heads * kHeadDim;
  const int64_t so = token_offset(t, a.src_page_shift, a.src_page_stride, a.src_bt, slot_stride);
  const int64_t dof = token_offset(r, a.dst_page_shift, a.dst_page_stride, a.dst_bt, slot_stride);
  const int per_layer = slot_stride / 8;
  const int items = a.n_layers * per_layer;
  const int i0 = (int)((int64_t)part * items / a.parts);
  const int i1 = (int)((int64_t)(part + 1) * items / a.parts);
  for (int it = i0 + tid; it < i1; it += kCompactThreads) {
    const int layer = it / per_layer;
    const int64_t col = (int64_t)(it - layer * per_layer) * 8;
    const int64_t s0 = (int64_t)layer * a.src_layer_stride + so + col;
    const int64_t d0 = (int64_t)layer * a.dst_layer_stride + dof + col;
    *(uint4*)(a.dst_k + d0) = load_once(a.src_k + s0);
    *(uint4*)(a.dst_v + d0) = load_once(a.src_v + s0);
  }
  if (tid == 0 && part == 0) {
    if (a.evicted_tokens) a.evicted_tokens[r] = (int32_t)t;
    for (int m = 0; m < a.meta.n; ++m) {
      switch (a.meta.elem_bytes[m]) {
        case 1: ((uint8_t*)a.meta.dst[m])[r] = ((const uint8_t*)a.meta.src[m])[t]; break;
        case 2: ((uint16_t*)a.meta.dst[m])[r] = ((const uint16_t*)a.meta.src[m])[t]; break;
        case 4: ((uint32_t*)a.meta.dst[m])[r] = ((const uint32_t*)a.meta.src[m])[t]; break;
        default: ((uint64_t*)a.meta.dst[m])[r] = ((const uint64_t*)a.meta.src[m])[t]; break;
      }
    }
  }
}

// One row per ceil(items/256) workgroups, one 16-byte K and V chunk per thread, as the
// evicted-row gather: the copies of swaps and loads (device staging <-> cache slots).
__global__ __launch_bounds__(kCompactThreads) void move_rows_kernel(MoveArgs a) {
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x / a.parts;
  const int part = (int)(blockIdx.x % a.parts);
  const int64_t st = a.src_rows ? (int64_t)a.src_rows[r] : a.src_first + r;
  const int64_t dt = a.dst_rows ? (int64_t)a.dst_rows[r] : a.dst_first + r;
  if (st < 0 || st >= a.src_tokens || dt < 0 || dt >= a.dst_tokens) return;
  const int slot_stride = a.n_kv_heads * kHeadDim;
  const int64_t so = token_offset(st, a.src_page_shift, a.src_page_stride, a.src_bt, slot_stride);
  const int64_t dof = token_offset(dt, a.dst_page_shift, a.dst_page_stride, a.dst_bt, slot_stride);
  const int per_layer = slot_stride / 8;
  const int items = a.n_layers * per_layer;
  const int i0 = (int)((int64_t)part * items / a.parts);
  const int i1 = (int)((int64_t)(part + 1) * items / a.parts);
  for (int it = i0 + tid; it < i1; it += kCompactThreads) {
    const int layer = it / per_layer;
    const int64_t col = (int64_t)(it - layer * per_layer) * 8;
    const int64_t s0 = (int64_t)layer * a.src_layer_stride + so + col;
    const int64_t d0 = (int64_t)layer * a.dst_layer_stride + dof + col;
    *(uint4*)(a.dst_k + d0) = load_once(a.src_k + s0);
    *(uint4*)(a.dst_v + d0) = load_once(a.src_v + s0);
  }
  if (tid == 0 && part == 0) {
    const int64_t m0 = a.meta_first + r;
    for (int m = 0; m < a.meta.n; ++m) {
      switch (a.meta.elem_bytes[m]) {
        case 1: ((uint8_t*)a.meta.dst[m])[dt] = ((const uint8_t*)a.meta.src[m])[m0]; break;
        case 2: ((uint16_t*)a.meta.dst[m])[dt] = ((const uint16_t*)a.meta.src[m])[m0]; break;
        case 4: ((uint32_t*)a.meta.dst[m])[dt] = ((const uint32_t*)a.meta.src[m])[m0]; break;
        default: ((uint64_t*)a.meta.dst[m])[dt] = ((const uint64_t*)a.meta.src[m])[m0]; break;
      }
    }
  }
}

}  // namespace

// Workgroups per token for a plain K/V copy of `items` 16-byte chunk pairs: every thread
// moves at most one item, and many short workgroups keep HBM streaming.
static int copy_parts(int items) { return (items + kCompactThreads - 1) / kCompactThreads; }

hipError_t launch_gather_evicted(const EvictArgs& a0, hipStream_t s) {
  if (a0.count <= 0) return hipSuccess;
  EvictArgs a = a0;
  a.parts = copy_parts(a.n_layers * a.n_kv_heads * (kHeadDim / 8));
  const int64_t grid = a.count * a.parts;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (trace_on())
    trace_launch("gather_evicted grid=%lld block=%d  rows=%lld first=%lld parts=%d", (long long)grid, kCompactThreads,
                 (long long)a.count, (long long)a.first, a.parts);
  hipLaunchKernelGGL(gather_evicted_kernel, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_move_rows(const MoveArgs& a0, hipStream_t s) {
  if (a0.count <= 0) return hipSuccess;
  MoveArgs a = a0;
  a.parts = copy_parts(a.n_layers * a.n_kv_heads * (kHeadDim / 8));
  const int64_t grid = a.count * a.parts;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (trace_on())
    trace_launch("move_rows grid=%lld block=%d  rows=%lld parts=%d meta=%d", (long long)grid, kCompactThreads,
                 (long long)a.count, a.parts, a.meta.n);
  hipLaunchKernelGGL(move_rows_kernel, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a);
  return hipGetLastError();
}

// One workgroup per pair: each first locates its pair with three block-wide searches over
// the keep list (a chain of barriers and cached loads), so splitting a token over several
// workgroups, as the other copies do, would repeat that latency (measured slower).
hipError_t launch_tail_compact(const TailArgs& a, int64_t pairs, hipStream_t s) {
  if (pairs > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (trace_on())
    trace_launch("tail_compact grid=%lld block=%d  start=%lld budget=%lld", (long long)(pairs > 0 ? pairs : 1),
                 kCompactThreads, (long long)a.start, (long long)a.budget);
  hipLaunchKernelGGL(tail_compact_kernel, dim3((unsigned)(pairs > 0 ? pairs : 1)), dim3(kCompactThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_remap_table(const int32_t* bt, int32_t* bt_out, int32_t* freed, int64_t keep_pages,
                              int64_t prefix_pages, int64_t evict_pages, hipStream_t s) {
  const int64_t n = keep_pages > evict_pages ? keep_pages : evict_pages;
  if (n <= 0) return hipSuccess;
  if (trace_on())
    trace_launch("remap_table grid=%lld block=256  keep_pages=%lld prefix_pages=%lld evict_pages=%lld",
                 (long long)((n + 255) / 256), (long long)keep_pages, (long long)prefix_pages, (long long)evict_pages);
  hipLaunchKernelGGL(remap_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bt, bt_out, freed,
                     keep_pages, prefix_pages, evict_pages);
  return hipGetLastError();
}

hipError_t launch_remap_rows(const CompactArgs& a, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (trace_on()) trace_launch("remap_rows grid=%lld block=256  ranks=%lld", (long long)((n + 255) / 256), (long long)n);
  hipLaunchKernelGGL(remap_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

hipError_t launch_remap_pages(const int32_t* bt, int32_t* bt_out, const int32_t* keep, const int64_t* n_keep,
                              int64_t max_keep, int page_shift, int64_t n_pages_src, uint32_t* status,
                              hipStream_t s) {
  const int64_t pages = (max_keep + ((int64_t)1 << page_shift) - 1) >> page_shift;
  const int64_t n = pages > 1 ? pages : 1;             // at least one thread clears the status
  if (trace_on())
    trace_launch("remap_pages grid=%lld block=256  max_pages=%lld", (long long)((n + 255) / 256), (long long)pages);
  hipLaunchKernelGGL(remap_pages_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bt, bt_out, keep,
                     n_keep, max_keep, page_shift, n_pages_src, status);
  return hipGetLastError();
}

int compact_parts(int n_layers, int n_kv_heads) {
  const int items = n_layers * n_kv_heads * 8;
  return (items + kCompactThreads - 1) / kCompactThreads;
}

// A launch that writes well beyond what the 256 MB memory-side cache holds streams its
// stores past the caches (measured: 19.8 GB in-place segment move 3.65 -> 3.39 ms); a
// smaller one keeps plain stores, whose dirty lines the cache absorbs and writes back
// after the kernel (2,048 Qwen3-8B tokens, 302 MB written: 0.101 against 0.117 ms).
constexpr int64_t kStreamStoreBytes = 1LL << 30;

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const int64_t n = a.rank1 - a.rank0;
  if (n <= 0) return hipSuccess;
  const int64_t grid = n * a.parts;
  if (a.parts < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t written = n * a.n_layers * a.n_kv_heads * (int64_t)kHeadDim * 2 * 2;
  const bool nt = written > kStreamStoreBytes;
  const dim3 g((unsigned)grid), b(kCompactThreads);
  if (trace_on())
    trace_launch("compact grid=%lld block=%d  ranks=[%lld,%lld) parts=%d layers=%d kv_heads=%d store=%d stream_stores=%d",
                 (long long)grid, kCompactThreads, (long long)a.rank0, (long long)a.rank1, a.parts, a.n_layers,
                 a.n_kv_heads, a.ref_src_k != nullptr, (int)nt);
  if (a.ref_src_k) {
    if (nt) hipLaunchKernelGGL((compact_kernel<true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((compact_kernel<true, false>), g, b, 0, s, a);
  } else {
    if (nt) hipLaunchKernelGGL((compact_kernel<false, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((compact_kernel<false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ref_invalidate(int32_t* pos, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (trace_on()) trace_launch("ref_invalidate grid=%lld block=256  slots=%lld", (long long)((count + 255) / 256), (long long)count);
  hipLaunchKernelGGL(ref_invalidate_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, pos, count);
  return hipGetLastError();
}

}  // namespace kvs
