// Windowed attention mass on gfx950: the one dense contraction of the path.
//
// What is computed (MemDecay, Method: the attention a token receives from the window
// queries, a mean over layers and heads; ActKV Sec. 2.3 and 7.1: A = exp(q.k - LSE) recovered from the log-sum-exp;
// PACE Sec. 2: SnapKV's observation window):
//   for every layer l, KV head g and window row r = (window query w, query head h of
//   g's GQA group), s_rj = scale * <q_r, k_j> over keys j <= N - W + w;
//   pass 1: LSE_r = log sum_j exp(s_rj)   (per key chunk, combined afterwards)
//   pass 2, sum mode:  mass_part[l,g][j] = sum_r exp(s_rj - LSE_r)
//   pass 2, max mode (ActKV Sec. 7.1, Algorithm 3):
//          mass_part[l,g][j] = sum_w max_h exp(s_(w,h)j - LSE_(w,h))
//                            = sum_w exp(max_h (s_(w,h)j - LSE_(w,h)))
// Rows are ordered window-query major: r = w * RS + h_local, with RS = G in sum mode and
// RS = G rounded up to a power of two in max mode (rows with h_local >= G are padding:
// zero queries and an infinite LSE, so they contribute nothing).  A group then occupies
// RS consecutive, aligned rows, which the MFMA output layout keeps inside one lane or
// one lane pair, so the max costs a few v_max and at most one cross-half shuffle, and
// only one exponential per group is taken.
//
// Work decomposition: one workgroup per (layer, KV head, chunk of keys, group of at
// most 256 rows).  Its waves each own 32 of the rows and keep those rows' queries in
// registers as MFMA operands for the whole chunk.  64-key tiles of K (16 KiB) stream into a ring of LDS
// buffers by direct global->LDS 16-byte loads issued several tiles ahead, so HBM
// latency hides behind tiles of work and no VGPRs stage the data.  Rows are stored
// with an XOR swizzle of their 16-byte pieces, which keeps the loads coalesced (every
// 16 lanes read one 256-byte key row) and the fragment reads free of bank conflicts.
// Page addresses are wave-uniform: a wave-wide load covers 4 keys of one page.
//
// Inside a tile each wave works on 32-key halves with two accumulator sets: it computes
// the logits of one half (v_mfma_f32_32x32x16_bf16) while turning the previous half into
// exponentials, so that the matrix core and the vector ALU overlap instead of taking
// turns (pass 2's group-maximum variant keeps one set and relies on the other waves of
// the SIMD).  Logits stay in fp32 accumulators and are consumed in registers: nothing
// of size rows x N is stored.
//
// Exponentials use exp2 with the scale folded into c = scale * log2(e).  Pass 1 keeps
// a running reference per lane and row and rescales only when a half's sum would leave
// the safe range (the first half always does), so the steady state costs one fma, one
// exp and one add per logit.  All reductions have a fixed order: results do not depend
// on scheduling.
#include "kv_internal.h"

namespace kvs {

namespace {

constexpr int kStages = 4;                          // K tiles resident in LDS
constexpr int kAhead = kStages - 1;                 // prefetch distance in tiles
static_assert(kStages >= 3, "a stage is refilled one barrier after its last read");
constexpr int kRowBytes = kHeadDim * 2;             // 256 B per key row
constexpr int kTileBytes = kTile * kRowBytes;       // 16 KiB
constexpr int kLoadsPerTile = kTileBytes / 1024;    // wave-wide 16-byte loads per tile

// s_waitcnt immediate for gfx9: vmcnt <= vm, lgkmcnt <= lgkm, expcnt unconstrained.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Compiler-only fence: keeps LDS accesses on their side of a hand-placed barrier.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a location in a __shared__ array (computed once per kernel: the
// conversion from a generic pointer costs vector instructions).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

// 16-byte global -> LDS load of every lane: lane L's 16 bytes land at lds + 16*L.  It is
// issued from inline assembly so that the compiler does not track it: otherwise it
// would conservatively wait for these loads before every LDS read, which would undo the
// prefetch.  Completion is awaited explicitly with vmcnt before the barrier that
// publishes a tile (all waits in this file are hand-placed for that reason).
// kNt marks the load non-temporal ("nt"): it streams through the caches instead of
// allocating in them.  Each pass reads every key once.  Pass 1 streams (measured: pass 1
// 1.2% faster, and pass 2 0.3% faster too); pass 2 keeps the keys it reads cached, as the
// compaction that follows re-reads the kept keys, and streaming there too would make
// compaction 19% slower for another 1.0% on pass 2.
template <bool kNt>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  // M0 carries the LDS destination; the previous M0 is restored so that the compiler's
  // own view of M0 stays valid.  The wait state separates the M0 write from its use.
  if constexpr (kNt)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(dst)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(dst)
        : "memory");
}

// Everything a workgroup needs to locate its keys and queries.  The G*W rows of one
// (layer, KV head) are split into groups of at most 256 rows, one workgroup each; wave
// wv owns rows row0 + 32*wv .. row0 + 32*wv + 31 of its group.  kNt: the key loads are
// non-temporal (see dma16).
template <int NW, bool kNt>
struct Ctx {
  static constexpr int LPW = (kLoadsPerTile + NW - 1) / NW;  // loads per wave per tile
  static constexpr bool kJunk = (kLoadsPerTile % NW) != 0;

  const ScoreArgs& a;
  int lane, wv, chunk_id, rs, row0, g, layer, lg, n_tiles, n_full, slot_stride;
  int64_t j0, j1;
  const uint16_t* kbase;
  int fo0;                        // per-lane LDS byte offset of K fragment ks = 0; the
                                  // fragment of k-step ks sits at fo0 ^ (ks << 5)
  int voff[LPW];                  // per-lane element offsets of this wave's loads in a page

  __device__ Ctx(const ScoreArgs& args) : a(args) {
    lane = threadIdx.x & 63;
    wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bid = blockIdx.x;
    chunk_id = bid % a.n_chunks;
    bid /= a.n_chunks;
    rs = bid % a.n_rsplit;
    bid /= a.n_rsplit;
    row0 = rs * kRowsPerGroup;
    g = bid % a.n_kv_heads;
    layer = bid / a.n_kv_heads;
    lg = layer * a.n_kv_heads + g;
    j0 = (int64_t)chunk_id * a.chunk;
    j1 = j0 + a.chunk < a.n_tokens ? j0 + a.chunk : a.n_tokens;
    n_tiles = (int)((j1 - j0 + kTile - 1) / kTile);
    n_full = a.page_shift >= 2 ? (int)((j1 - j0) / kTile) : 0;
    slot_stride = a.n_kv_heads * kHeadDim;
    kbase = a.k + (int64_t)layer * a.layer_stride + g * kHeadDim;
    // key row kk = 32*kb + lane%32 holds dims 16*ks + 8*(lane/32) in piece
    // c16 = 2*ks + lane/32, stored at piece slot c16 ^ (kk % 16)
    // piece slot (2*ks + lane/32) ^ (lane%16) = ((lane/32) ^ (lane%16)) ^ 2*ks, so the
    // k-step only flips bits 5..7 of the byte offset
    fo0 = (lane & 31) * kRowBytes + (((lane >> 5) ^ (lane & 15)) << 4);
#pragma unroll
    for (int m = 0; m < LPW; ++m) {
      const int row = 4 * load_slot(m) + (lane >> 4);
      voff[m] = (lane >> 4) * slot_stride + (((lane & 15) ^ (row & 15)) << 3);
    }
  }

  // Query row row0 + 32*wv + lane%32 as 32x32x16 fragments: dims 16*ks + 8*(lane/32).
  // Padding rows (past the last row, or h_local >= G) get zero queries.
  __device__ void load_queries(bf16x8 (&qf)[8]) const {
    const int W = a.window;
    const int row = row0 + wv * 32 + (lane & 31);
    const int w = row / a.row_stride;
    const int hl = row - w * a.row_stride;
    if (row < a.rows && hl < a.group) {
      const int h = g * a.group + hl;
      const uint16_t* qp =
          a.q + (((int64_t)layer * W + w) * a.n_q_heads + h) * kHeadDim + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = bf16x8{};
    }
  }

  // Load slots of this wave: wave wv fills rows 4*LPW*wv .. 4*LPW*(wv+1)-1 of a tile,
  // 4 rows per wave-wide load.  When 16 is not a multiple of NW the surplus loads of
  // the last waves go to a junk buffer, so every wave has the same number in flight.
  __device__ __forceinline__ int load_slot(int m) const {
    const int i = wv * LPW + m;
    return kJunk && i >= kLoadsPerTile ? kLoadsPerTile - 1 : i;
  }

  // Tile t is full (all 64 keys before the chunk end) and its pages are wave-uniform.
  __device__ __forceinline__ bool uniform_tile(int t) const { return t < n_full; }

  // Physical pages of this wave's loads of tile t (scalar loads, issued one iteration
  // before they are needed so that their latency hides behind a tile of work).
  __device__ __forceinline__ void fetch_pages(int t, const int32_t* __restrict__ bt,
                                              int32_t (&ph)[LPW]) const {
    if (!uniform_tile(t)) return;
    const uint32_t tile_j0 = (uint32_t)j0 + (uint32_t)t * (uint32_t)kTile;   // N < 2^31
#pragma unroll
    for (int m = 0; m < LPW; ++m) ph[m] = (int32_t)((tile_j0 + 4u * (uint32_t)load_slot(m)) >> a.page_shift);
    if (bt) {
#pragma unroll
      for (int m = 0; m < LPW; ++m) ph[m] = bt[ph[m]];
    }
  }

  // Loads of a full tile whose pages are wave-uniform (page size >= 4): the per-lane part
  // of every address is precomputed.
  // kScalar: page ids are re-read as scalars first (the stage-unrolled loops need this
  // to keep the page arithmetic off the vector ALU).
  template <bool kScalar = false>
  __device__ __forceinline__ void issue_fast(int t, uint32_t stage, uint32_t junk,
                                             const int32_t (&ph)[LPW]) const {
    // 32-bit pieces: the page stride is below 2^32 elements and the in-page offset small
    const uint32_t tj_lo = (uint32_t)j0 + (uint32_t)t * (uint32_t)kTile;
    const uint32_t pmask = (1u << a.page_shift) - 1u;
    const uint32_t pstride = (uint32_t)a.page_stride;
#pragma unroll
    for (int m = 0; m < LPW; ++m) {
      const int i = load_slot(m);
      const uint32_t dst = kJunk && wv * LPW + m >= kLoadsPerTile ? junk : stage + i * 1024;
      const uint32_t page = (uint32_t)(kScalar ? __builtin_amdgcn_readfirstlane(ph[m]) : ph[m]);
      const uint64_t poff = (uint64_t)page * pstride;
      const uint32_t inpage = ((tj_lo + 4u * (uint32_t)i) & pmask) * (uint32_t)slot_stride;
      const uint16_t* base = kbase + poff + inpage;
      dma16<kNt>(base + voff[m], dst);
    }
  }

  // Issue this wave's direct-to-LDS loads of tile t into `stage`.  Load slot i fills
  // rows 4i..4i+3; lane L carries piece (L%16) ^ (row%16) of row 4i + L/16, so it lands
  // in swizzled position.  Keys past the chunk end are clamped to the last valid key
  // (their logits are masked later).
  __device__ void issue_tile(int t, uint32_t stage, uint32_t junk, const int32_t* __restrict__ bt,
                             const int32_t (&ph)[LPW]) const {
    const int64_t tile_j0 = j0 + (int64_t)t * kTile;
    if (uniform_tile(t)) {
      // a wave-wide load reads 4 keys of one page: the page address is wave-uniform
      const int64_t pmask = (1LL << a.page_shift) - 1;
#pragma unroll
      for (int m = 0; m < LPW; ++m) {
        const int i = load_slot(m);
        const uint32_t dst = kJunk && wv * LPW + m >= kLoadsPerTile ? junk : stage + i * 1024;
        const int row = 4 * i + (lane >> 4);
        const int c16 = (lane & 15) ^ (row & 15);
        const uint16_t* base =
            kbase + (int64_t)ph[m] * a.page_stride + ((tile_j0 + 4 * i) & pmask) * slot_stride;
        dma16<kNt>(base + (lane >> 4) * slot_stride + c16 * 8, dst);
      }
    } else {
      // small pages or the chunk's ragged last tile: per-lane addresses
#pragma unroll
      for (int m = 0; m < LPW; ++m) {
        const int i = load_slot(m);
        const uint32_t dst = kJunk && wv * LPW + m >= kLoadsPerTile ? junk : stage + i * 1024;
        const int row = 4 * i + (lane >> 4);
        const int c16 = (lane & 15) ^ (row & 15);
        int64_t j = tile_j0 + row;
        if (j >= j1) j = j1 - 1;
        const uint16_t* src =
            kbase + token_offset(j, a.page_shift, a.page_stride, bt, slot_stride) + c16 * 8;
        dma16<kNt>(src, dst);
      }
    }
  }

  // Wait until at most `pending` tiles of this wave's loads are still in flight (the
  // newest ones), make this wave's LDS writes visible, then synchronise the workgroup.
  __device__ __forceinline__ void wait_and_barrier(int pending) const {
    compiler_fence();
    static_assert(kAhead <= 5, "wait cases below cover up to 4 pending tiles");
    switch (pending) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_imm(LPW, 0)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LPW, 0)); break;
      case 3: __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * LPW, 0)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * LPW, 0)); break;
    }
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }

  // K fragment of half `half` (keys 32*half + lane%32), dims 16*ks + 8*(lane/32).
  __device__ __forceinline__ bf16x8 key_frag(const uint8_t* tile, int half, int ks) const {
    return *(const bf16x8*)(tile + half * 32 * kRowBytes + (fo0 ^ (ks << 5)));
  }
};

template <int V>
struct StageC {
  static constexpr int value = V;
};

// --------------------------------------------------------------------------- pipeline
// The tile loop shared by both passes.  Pass P provides mma(tile, half, acc) (the
// logits of one 32-key half), consume<kMask>(acc, half_j0, half, cb) (the VALU work on
// them), between(t, cb) (after the barrier that closes tile t's partials) and finish().
// The steady-state loops cover tiles that are full, visible to every row and loaded
// through the fast page path; the remaining tiles take a general loop with every check
// in place.  Column buffer cb of tile t is t % 3.
//
// P::kOverlap: each wave computes the logits of the next half while the previous half
// goes through exp (two accumulator sets), so one wave keeps both the matrix core and
// the vector ALU busy.  Otherwise each half runs MFMA then exp with one accumulator
// set and the overlap comes from the other waves resident on the SIMD.
// The steady-state loop takes one step per ring stage (tile t uses stage t % kStages),
// so every LDS fragment address is a constant offset from a per-lane base and needs no
// address arithmetic.  P::enter_steady() runs once before that loop, and its consume
// calls pass kRegNl = true.
template <int NW, bool kNt, class P>
__device__ __forceinline__ void run_tiles(const Ctx<NW, kNt>& x, P& p, uint8_t (*kt)[kTileBytes],
                                          uint8_t* junk, const int32_t* __restrict__ bt) {
  const int nt = x.n_tiles;
  // LDS addresses of the ring stages and the junk buffer, for the direct-to-LDS loads
  const uint32_t kt0 = lds_addr(kt[0]);
  const uint32_t jk = lds_addr(junk);
  auto stage_addr = [&](int s) { return kt0 + (uint32_t)s * (uint32_t)kTileBytes; };
  const int nf = x.n_full;  // full tiles (all 64 keys before the chunk end), wave-uniform pages
  // clean tiles: full and every key visible to every window row
  const int64_t last_clean_key = x.a.n_tokens - x.a.window;
  const int64_t clean_end = x.j1 < last_clean_key + 1 ? x.j1 : last_clean_key + 1;
  const int nc = clean_end > x.j0 ? (int)((clean_end - x.j0) / kTile) : 0;

  int32_t ph[Ctx<NW, kNt>::LPW] = {};
  for (int t = 0; t < kAhead && t < nt; ++t) {
    x.fetch_pages(t, bt, ph);
    x.issue_tile(t, stage_addr(t), jk, bt, ph);
  }
  if (kAhead < nt) x.fetch_pages(kAhead, bt, ph);
  x.wait_and_barrier((nt < kAhead ? nt : kAhead) - 1);

  // hidden keys exist only in halves that reach past the last clean key or the chunk end
  auto masked = [&](int64_t hj) { return hj + 31 > last_clean_key || hj + 32 > x.j1; };
  int t = 0, st = 0, cb = 0;  // tile, its LDS stage, its column buffer
  if constexpr (P::kOverlap) {
    f32x16 acc0, acc1;
    p.mma(kt[0], 0, acc0);
    // one step per ring stage (tile t uses stage t % kStages): every LDS fragment
    // address is a constant offset from a per-lane base
    auto step = [&](auto stage) -> bool {
      constexpr int ST = decltype(stage)::value;
      constexpr int ST1 = (ST + 1) % kStages, STA = (ST + kStages - 1) % kStages;
      t = __builtin_amdgcn_readfirstlane(t);   // uniform: keeps the tile arithmetic scalar
      if (!(t + kAhead < nf && t < nc)) return false;
      const int64_t tj = x.j0 + (int64_t)t * kTile;
      const int cbp = cb == 0 ? 2 : cb - 1;
      x.template issue_fast<true>(t + kAhead, kt0 + STA * kTileBytes, jk, ph);
      if (t + kAhead + 1 < nt) x.fetch_pages(t + kAhead + 1, bt, ph);
      p.mma(kt[ST], 1, acc1);
      p.template consume<false, true>(acc0, tj, 0, cb);
      x.wait_and_barrier(kAhead - 1);
      if (t >= 1) p.between(t - 1, cbp);
      p.mma(kt[ST1], 0, acc0);
      p.template consume<false, true>(acc1, tj + 32, 1, cb);
      ++t;
      cb = cb == 2 ? 0 : cb + 1;
      return true;
    };
    static_assert(kStages == 4, "the unrolled steady loop has one step per stage");
    p.enter_steady();
    while (step(StageC<0>{}) && step(StageC<1>{}) && step(StageC<2>{}) && step(StageC<3>{})) {
    }
    st = t % kStages;
    for (; t < nt; ++t) {
      t = __builtin_amdgcn_readfirstlane(t);   // uniform: keeps the tile arithmetic scalar
      const int64_t tj = x.j0 + (int64_t)t * kTile;
      const int st1 = st == kStages - 1 ? 0 : st + 1;
      const int sta = st == 0 ? kStages - 1 : st - 1;
      const int cbp = cb == 0 ? 2 : cb - 1;
      if (t + kAhead < nt) x.issue_tile(t + kAhead, stage_addr(sta), jk, bt, ph);
      if (t + kAhead + 1 < nt) x.fetch_pages(t + kAhead + 1, bt, ph);
      p.mma(kt[st], 1, acc1);
      if (masked(tj)) p.template consume<true>(acc0, tj, 0, cb);
      else p.template consume<false>(acc0, tj, 0, cb);
      // tile t+1 must be resident; tiles t+2 .. t+kAhead may still be loading
      const int issued = t + kAhead < nt ? t + kAhead : nt - 1;
      x.wait_and_barrier(issued - (t + 1) > 0 ? issued - (t + 1) : 0);
      if (t >= 1) p.between(t - 1, cbp);
      if (t + 1 < nt) p.mma(kt[st1], 0, acc0);
      if (masked(tj + 32)) p.template consume<true>(acc1, tj + 32, 1, cb);
      else p.template consume<false>(acc1, tj + 32, 1, cb);
      st = st1;
      cb = cb == 2 ? 0 : cb + 1;
    }
    x.wait_and_barrier(0);
    p.between(nt - 1, cb == 0 ? 2 : cb - 1);
  } else {
    f32x16 acc;
    // Steady state, one step per ring stage (tile t uses stage t % kStages): every LDS
    // fragment address is then a constant offset from a per-lane base, which saves the
    // address arithmetic of each read.
    auto step = [&](auto stage) -> bool {
      constexpr int ST = decltype(stage)::value;
      constexpr int STA = (ST + kStages - 1) % kStages;
      if (!(t + kAhead < nf && t < nc)) return false;
      const int64_t tj = x.j0 + (int64_t)t * kTile;
      x.issue_fast(t + kAhead, kt0 + STA * kTileBytes, jk, ph);
      if (t + kAhead + 1 < nt) x.fetch_pages(t + kAhead + 1, bt, ph);
      p.mma(kt[ST], 0, acc);
      p.template consume<false, true>(acc, tj, 0, cb);
      p.mma(kt[ST], 1, acc);
      p.template consume<false, true>(acc, tj + 32, 1, cb);
      x.wait_and_barrier(kAhead - 1);
      p.between(t, cb);
      ++t;
      cb = cb == 2 ? 0 : cb + 1;
      return true;
    };
    static_assert(kStages == 4, "the unrolled steady loop has one step per stage");
    p.enter_steady();
    while (step(StageC<0>{}) && step(StageC<1>{}) && step(StageC<2>{}) && step(StageC<3>{})) {
    }
    st = t % kStages;
    for (; t < nt; ++t) {
      const int64_t tj = x.j0 + (int64_t)t * kTile;
      const int sta = st == 0 ? kStages - 1 : st - 1;
      if (t + kAhead < nt) x.issue_tile(t + kAhead, stage_addr(sta), jk, bt, ph);
      if (t + kAhead + 1 < nt) x.fetch_pages(t + kAhead + 1, bt, ph);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int64_t hj = tj + 32 * half;
        p.mma(kt[st], half, acc);
        if (masked(hj)) p.template consume<true>(acc, hj, half, cb);
        else p.template consume<false>(acc, hj, half, cb);
      }
      const int issued = t + kAhead < nt ? t + kAhead : nt - 1;
      x.wait_and_barrier(issued - (t + 1) > 0 ? issued - (t + 1) : 0);
      p.between(t, cb);
      st = st == kStages - 1 ? 0 : st + 1;
      cb = cb == 2 ? 0 : cb + 1;
    }
  }
  p.finish();
}

// --------------------------------------------------------------------------- pass 1
// S^T = K Q^T: each lane holds one query row (row0 + 32*wv + lane%32) against 16 keys of
// a half (8*(i/4) + 4*(lane/32) + i%4), so the running softmax state is lane-local.
// Element i of a lane's 32x32 MFMA block sits at offset 8*(i/4) + i%4 from the lane's
// first row or key; the number of these offsets below l, for 0 <= l <= 32.
__device__ __forceinline__ int offsets_below(int l) {
  const int r = l & 7;
  return 4 * (l >> 3) + (r < 4 ? r : 4);
}

template <int NW>
struct LsePass {
  using C = Ctx<NW, true>;
  static constexpr bool kOverlap = true;
  const C& x;
  const bf16x8 (&qf)[8];
  float c;
  int last_key;                   // last key this lane's row may see (rows are below 2^31 keys)
  float m, l;
  float nm;                       // -m, kept so that the exponent argument is one fma

  __device__ LsePass(const C& ctx, const bf16x8 (&q)[8]) : x(ctx), qf(q) {
    c = x.a.c;
    const int w = (x.row0 + x.wv * 32 + (x.lane & 31)) / x.a.row_stride;
    last_key = (int)(x.a.n_tokens - x.a.window) + w;
    m = -1e30f;
    nm = 1e30f;
    l = 0.f;
  }

  __device__ __forceinline__ void mma(const uint8_t* tile, int half, f32x16& acc) const {
    acc = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < 8; k0 += 4) {
      bf16x8 kf[8];
#pragma unroll
      for (int ks = k0; ks < k0 + 4; ++ks) kf[ks] = x.key_frag(tile, half, ks);
#pragma unroll
      for (int ks = k0; ks < k0 + 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], acc, 0, 0, 0);
    }
  }

  // Bit i set when element i is a key this lane's row must not see (past the chunk
  // end, or after the row's own position).
  // Element i holds key base + off_i (base = half_j0 + 4*(lane/32), off_i = 8*(i/4) +
  // i%4), and the row sees keys below min(chunk end, last_key + 1): one 32-bit limit.
  __device__ uint32_t hidden(int64_t half_j0) const {
    const int base = (int)half_j0 + 4 * (x.lane >> 5);
    const int end = (int)x.j1 < last_key + 1 ? (int)x.j1 : last_key + 1;
    int l = end - base;
    l = l < 0 ? 0 : (l > 32 ? 32 : l);
    // the offsets increase with i, so the hidden elements are the ones from the count of
    // offsets below l on
    return (0xFFFFu << offsets_below(l)) & 0xFFFFu;
  }

  // Sum of 2^(c*s + nref) over the half, nref = -reference; hidden keys are excluded
  // through their exponent argument (the accumulators are only read, never rewritten).
  template <bool kMask>
  __device__ __forceinline__ float sums(const f32x16& acc, uint32_t h, float nref) const {
    float r[4];                                      // four running partial sums
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arg = __builtin_fmaf(acc[i], c, nref);
      if (kMask && ((h >> i) & 1u)) arg = -INFINITY;
      const float e = exp2f_fast(arg);
      r[i & 3] = i < 4 ? e : r[i & 3] + e;
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
  }

  __device__ __forceinline__ void enter_steady() {}

  // Fold a half into the running state, rescaling when its sum left [0, 2^64].
  template <bool kMask, bool = false>
  __device__ __forceinline__ void consume(const f32x16& acc, int64_t half_j0, int, int) {
    const uint32_t h = kMask ? hidden(half_j0) : 0u;
    float ts = sums<kMask>(acc, h, nm);
    if (__builtin_amdgcn_ballot_w64(!(ts <= 0x1p64f)) != 0) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!kMask || !((h >> i) & 1u)) tmax = fmaxf(tmax, acc[i] * c);
      const float mn = fmaxf(m, tmax);
      l *= exp2f_fast(m - mn);
      m = mn;
      nm = -mn;
      ts = sums<kMask>(acc, h, nm);
    }
    l += ts;
  }

  __device__ __forceinline__ void between(int, int) {}

  // combine the two lanes holding the same query (lane, lane^32) and store the chunk's
  // (max, sum) of the row
  __device__ void finish() {
    const float mo = __shfl_xor(m, 32);
    const float lo = __shfl_xor(l, 32);
    const float mn = fmaxf(m, mo);
    const float ln = l * exp2f_fast(m - mn) + lo * exp2f_fast(mo - mn);
    const int row = x.row0 + x.wv * 32 + x.lane;
    if (x.lane < 32 && row < x.a.rows)
      x.a.lse_part[((int64_t)x.lg * x.a.n_chunks + x.chunk_id) * x.a.rows + row] = make_float2(mn, ln);
  }
};

// Two workgroups per CU need ceil(2*NW/4) waves per SIMD: 3 for five or six waves (at
// most 168 VGPRs per lane), 4 for eight (at most 128).  amdgpu_waves_per_eu makes the
// register allocator honour that; smaller workgroups are bound by LDS instead.

template <int NW>
__device__ __forceinline__ void lse_pass_body(const ScoreArgs& a, const int32_t* __restrict__ bt) {
  using C = Ctx<NW, true>;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[kStages][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t junk[C::kJunk ? 1024 : 16];
  const C x(a);
  bf16x8 qf[8];
  x.load_queries(qf);
  LsePass<NW> p(x, qf);
  run_tiles(x, p, kt, junk, bt);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void lse_pass_kernel(ScoreArgs a, const int32_t* __restrict__ bt) {
  lse_pass_body<NW>(a, bt);
}
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void lse_pass_kernel_3w(
    ScoreArgs a, const int32_t* __restrict__ bt) {
  lse_pass_body<NW>(a, bt);
}
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void lse_pass_kernel_4w(
    ScoreArgs a, const int32_t* __restrict__ bt) {
  lse_pass_body<NW>(a, bt);
}

// --------------------------------------------------------------------------- pass 2
// S = Q K^T: each lane holds one key of a half (32*half + lane%32) against 16 rows
// (row0 + 32*wv + 8*(i/4) + 4*(lane/32) + i%4), so the per-key row sums are lane-local.
// LSE (log2 units) of row `row` of (layer, KV head) lg: its per-chunk (max, sum) partials
// combined in float64 in chunk order, or the caller's natural-log LSE; +inf for a padding
// row of the group maximum (weight exp(-inf) = 0).  *nat: the row's [L][Hq][W] index, or
// -1 for a padding row.
__device__ __forceinline__ float row_lse2(const CombineArgs& a, int lg, int row, int64_t* nat) {
  const int layer = lg / a.n_kv_heads;
  const int g = lg - layer * a.n_kv_heads;
  const int w = row / a.row_stride;
  const int hl = row - w * a.row_stride;
  if (hl >= a.group) {
    *nat = -1;
    return INFINITY;
  }
  const int h = g * a.group + hl;
  *nat = ((int64_t)layer * a.n_q_heads + h) * a.window + w;
  if (a.lse_in) return (float)((double)a.lse_in[*nat] * 1.4426950408889634);
  // partials are read 8 chunks at a time so that their loads are in flight together;
  // the maximum and the chunk-ordered float64 sum are unchanged by the batching
  const float2* p = a.lse_part + (int64_t)lg * a.n_chunks * a.rows + row;
  constexpr int kB = 8;
  float mx = -1e30f;
  for (int ch0 = 0; ch0 < a.n_chunks; ch0 += kB) {
    float x[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) x[u] = ch0 + u < a.n_chunks ? p[(int64_t)(ch0 + u) * a.rows].x : -1e30f;
#pragma unroll
    for (int u = 0; u < kB; ++u) mx = fmaxf(mx, x[u]);
  }
  double sum = 0.0;
  for (int ch0 = 0; ch0 < a.n_chunks; ch0 += kB) {
    float2 v[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u)
      v[u] = ch0 + u < a.n_chunks ? p[(int64_t)(ch0 + u) * a.rows] : make_float2(-1e30f, 0.f);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (ch0 + u < a.n_chunks) sum += (double)v[u].y * exp2((double)v[u].x - (double)mx);
  }
  return (float)((double)mx + log2(sum));
}

// Each lane leaves its partial in LDS; after the barrier that closes the tile 64
// threads add the 2*NW partials of each key in a fixed order and store the tile's
// column sums (three column buffers rotate between tiles).
// kMaxLog = 0: sum over rows.  kMaxLog = m > 0: max over aligned groups of 2^m rows
// first (RS = 2^m), one exponential per group.
template <int NW, int kMaxLog>
struct MassPass {
  using C = Ctx<NW, false>;
  // the sum keeps two accumulator sets (the group maximum's extra registers would spill)
  static constexpr bool kOverlap = kMaxLog == 0;
  static constexpr int kColStride = 2 * NW + 1;     // floats per key (partials + pad)
  const C& x;
  const bf16x8 (&qf)[8];
  float (*colp)[kTile * kColStride];
  const float* nlw;                                  // -LSE2 of this wave's 32 rows (LDS)
  float c;
  float nl_[16];                                     // this lane's 16 rows' -LSE2, held in
                                                     // registers over the steady loop

  // nls: LDS block of NW*32 floats; each wave stores -LSE2 of its rows (-inf past the
  // last row).  Only the owning wave reads them, so no barrier is needed.
  __device__ MassPass(const C& ctx, const bf16x8 (&q)[8], float (*cp)[kTile * kColStride],
                      float* nls)
      : x(ctx), qf(q), colp(cp) {
    c = x.a.c;
    float* own = nls + x.wv * 32;
    if (x.lane < 32) {
      const int row = x.row0 + x.wv * 32 + x.lane;
      float nl = -INFINITY;
      if (row < x.a.rows) {
        if (x.a.fuse_combine) {
          // a small grid combines its rows' chunk partials itself, with the arithmetic of
          // lse_combine_kernel; the workgroup of chunk 0 also writes the caller's LSE
          int64_t nat;
          const float l2 = row_lse2(x.a.comb, x.lg, row, &nat);
          if (x.chunk_id == 0 && nat >= 0 && x.a.comb.lse_out)
            x.a.comb.lse_out[nat] = (float)((double)l2 * 0.6931471805599453);
          nl = -l2;
        } else {
          nl = -x.a.lse2[(int64_t)x.lg * x.a.rows + row];
        }
      }
      own[x.lane] = nl;
    }
    // the status word is cleared before the epilogue, later on the stream, sets bits
    if (x.a.fuse_combine && blockIdx.x == 0 && threadIdx.x == 0 && x.a.comb.status) *x.a.comb.status = 0u;
    nlw = own;
  }

  // The steady loop takes every row's -LSE2 from registers: reading them from LDS for
  // each half tile cost about 4% of the pass.  The other loops read them from LDS, so
  // that these registers are free there.
  __device__ __forceinline__ void enter_steady() { load_nl(nl_); }

  // -LSE2 of this lane's 16 rows 8*(i/4) + 4*(lane/32) + i%4, as four float4 reads
  __device__ __forceinline__ void load_nl(float (&nl)[16]) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 v = *(const float4*)(nlw + 8 * g + 4 * (x.lane >> 5));
      nl[4 * g] = v.x;
      nl[4 * g + 1] = v.y;
      nl[4 * g + 2] = v.z;
      nl[4 * g + 3] = v.w;
    }
  }

  __device__ __forceinline__ void mma(const uint8_t* tile, int half, f32x16& acc) const {
    acc = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < 8; k0 += 4) {
      bf16x8 kf[8];
#pragma unroll
      for (int ks = k0; ks < k0 + 4; ++ks) kf[ks] = x.key_frag(tile, half, ks);
#pragma unroll
      for (int ks = k0; ks < k0 + 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf[ks], acc, 0, 0, 0);
    }
  }

  // Bit i set when row i of this lane must not see its key (past the chunk end, or
  // after the row's own position).
  // Row r (window query w = r / row_stride) sees key j when j <= N - W + w, i.e. when
  // w >= d = j - (N - W), i.e. when r >= d * row_stride.  Element i holds row
  // rbase + off_i (rbase = row0 + 32*wv + 4*(lane/32), off_i = 8*(i/4) + i%4), so one
  // 32-bit limit decides all 16 elements (d is clamped to [0, W]: all rows see the key
  // below 0, none of the real rows above W).
  __device__ uint32_t hidden(int64_t half_j0) const {
    const int64_t j = half_j0 + (x.lane & 31);
    if (j >= x.j1) return 0xFFFFu;
    const int64_t d64 = j - (x.a.n_tokens - x.a.window);
    const int d = d64 < 0 ? 0 : (d64 > x.a.window ? x.a.window : (int)d64);
    int lim = d * x.a.row_stride - (x.row0 + x.wv * 32 + 4 * (x.lane >> 5));
    lim = lim < 0 ? 0 : (lim > 32 ? 32 : lim);
    return (1u << offsets_below(lim)) - 1u;   // the offsets increase with i
  }

  // This lane's share of the column sum of one half: hidden entries are excluded by
  // their exponent argument (the accumulators are only read, never rewritten).
  // kRegNl: -LSE2 from the registers loaded by enter_steady, else from LDS.
  template <bool kMask, bool kRegNl = false>
  __device__ __forceinline__ void consume(const f32x16& acc, int64_t half_j0, int half, int cb) const {
    const uint32_t h = kMask ? hidden(half_j0) : 0u;
    float part;
    if constexpr (kMaxLog == 0) {
      float r[4];                                    // four running partial sums
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float nv[4];
        if constexpr (kRegNl) {
#pragma unroll
          for (int u = 0; u < 4; ++u) nv[u] = nl_[4 * g + u];
        } else {
          // four rows at a time, to keep few registers live beside the second
          // accumulator set
          const float4 v = *(const float4*)(nlw + 8 * g + 4 * (x.lane >> 5));
          nv[0] = v.x;
          nv[1] = v.y;
          nv[2] = v.z;
          nv[3] = v.w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * g + u;
          float arg = __builtin_fmaf(acc[i], c, nv[u]);
          if (kMask && ((h >> i) & 1u)) arg = -INFINITY;
          const float e = exp2f_fast(arg);
          r[u] = g == 0 ? e : r[u] + e;
        }
      }
      part = (r[0] + r[1]) + (r[2] + r[3]);
    } else {
      float nl[16];
      if constexpr (kRegNl) {
#pragma unroll
        for (int i = 0; i < 16; ++i) nl[i] = nl_[i];
      } else {
        load_nl(nl);
      }
      float arg[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        arg[i] = __builtin_fmaf(acc[i], c, nl[i]);
        if (kMask && ((h >> i) & 1u)) arg[i] = -INFINITY;
      }
      part = group_max_sum(arg);
    }
    colp[cb][(32 * half + (x.lane & 31)) * kColStride + 2 * x.wv + (x.lane >> 5)] = part;
  }

  // Sum over this lane's groups of exp2(max of the group's arguments).  Element i holds
  // row 8*(i/4) + 4*(lane/32) + i%4 of the wave's 32: groups of 2 and 4 rows lie inside
  // the lane; a group of 8, 16 or 32 rows spans both halves of the lane pair
  // (lane, lane ^ 32), which exchange their partial maxima once and split the groups
  // between them (for 32 rows the upper lane contributes 0).
  __device__ __forceinline__ float group_max_sum(const float (&arg)[16]) const {
    if constexpr (kMaxLog == 1) {
      float r[4];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float e = exp2f_fast(fmaxf(arg[2 * p], arg[2 * p + 1]));
        r[p & 3] = p < 4 ? e : r[p & 3] + e;
      }
      return (r[0] + r[1]) + (r[2] + r[3]);
    } else {
      float v[4];                                    // max over rows 8m + 4*(lane/32) + 0..3
#pragma unroll
      for (int m = 0; m < 4; ++m)
        v[m] = fmaxf(fmaxf(arg[4 * m], arg[4 * m + 1]), fmaxf(arg[4 * m + 2], arg[4 * m + 3]));
      if constexpr (kMaxLog == 2) {
        return (exp2f_fast(v[0]) + exp2f_fast(v[1])) + (exp2f_fast(v[2]) + exp2f_fast(v[3]));
      } else {
        const bool upper = x.lane >= 32;
        if constexpr (kMaxLog == 3) {
          // lower lane finishes groups 0 and 1, upper lane groups 2 and 3
          const float r0 = __shfl_xor(upper ? v[0] : v[2], 32);
          const float r1 = __shfl_xor(upper ? v[1] : v[3], 32);
          const float g0 = fmaxf(upper ? v[2] : v[0], r0);
          const float g1 = fmaxf(upper ? v[3] : v[1], r1);
          return exp2f_fast(g0) + exp2f_fast(g1);
        } else if constexpr (kMaxLog == 4) {
          const float u0 = fmaxf(v[0], v[1]);        // rows 0..15
          const float u1 = fmaxf(v[2], v[3]);        // rows 16..31
          const float r = __shfl_xor(upper ? u0 : u1, 32);
          return exp2f_fast(fmaxf(upper ? u1 : u0, r));
        } else {
          static_assert(kMaxLog == 5, "groups of at most 32 rows");
          const float u = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
          const float r = __shfl_xor(u, 32);
          return upper ? 0.f : exp2f_fast(fmaxf(u, r));
        }
      }
    }
  }

  // 64 threads: column sums of finished tile t, partials added in a fixed order.
  __device__ __forceinline__ void between(int t, int cb) const {
    if (threadIdx.x < kTile) {
      const int64_t j = x.j0 + (int64_t)t * kTile + threadIdx.x;
      if (j < x.j1) {
        const float* q = colp[cb] + threadIdx.x * kColStride;
        float s = q[0];
#pragma unroll
        for (int k = 1; k < 2 * NW; ++k) s += q[k];
        x.a.mass_part[((int64_t)x.lg * x.a.n_rsplit + x.rs) * x.a.n_tokens + j] = s;
      }
    }
  }

  __device__ __forceinline__ void finish() const {}
};

template <int NW, int kMaxLog>
__device__ __forceinline__ void mass_pass_body(const ScoreArgs& a, const int32_t* __restrict__ bt) {
  using C = Ctx<NW, false>;
  using P = MassPass<NW, kMaxLog>;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[kStages][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t junk[C::kJunk ? 1024 : 16];
  __shared__ float colp[3][kTile * P::kColStride];
  __shared__ __attribute__((aligned(16))) float nls[NW * 32];
  const C x(a);
  bf16x8 qf[8];
  x.load_queries(qf);
  P p(x, qf, colp, nls);
  run_tiles(x, p, kt, junk, bt);
}

template <int NW, int kMaxLog>
__global__ __launch_bounds__(NW * 64) void mass_pass_kernel(ScoreArgs a, const int32_t* __restrict__ bt) {
  mass_pass_body<NW, kMaxLog>(a, bt);
}
template <int NW, int kMaxLog>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void mass_pass_kernel_3w(
    ScoreArgs a, const int32_t* __restrict__ bt) {
  mass_pass_body<NW, kMaxLog>(a, bt);
}
template <int NW, int kMaxLog>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void mass_pass_kernel_4w(
    ScoreArgs a, const int32_t* __restrict__ bt) {
  mass_pass_body<NW, kMaxLog>(a, bt);
}

// MODE < 0: LSE pass; MODE >= 0: mass pass with kMaxLog = MODE.
template <int MODE>
hipError_t launch_nw(const ScoreArgs& a, int nw, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_chunks * a.n_rsplit * a.n_kv_heads * a.n_layers));
  switch (nw) {
#define KVS_CASE(NWV, SUFFIX)                                                                        \
  case NWV:                                                                                           \
    if constexpr (MODE >= 0)                                                                          \
      hipLaunchKernelGGL((mass_pass_kernel##SUFFIX<NWV, (MODE < 0 ? 0 : MODE)>), grid, dim3(NWV * 64), \
                         0, s, a, a.block_table);                                                     \
    else                                                                                              \
      hipLaunchKernelGGL((lse_pass_kernel##SUFFIX<NWV>), grid, dim3(NWV * 64), 0, s, a, a.block_table);  \
    break;
    KVS_CASE(1, )
    KVS_CASE(2, )
    KVS_CASE(3, )
    KVS_CASE(4, )
    KVS_CASE(5, _3w)
    KVS_CASE(6, _3w)
    KVS_CASE(7, )
    KVS_CASE(8, _4w)
#undef KVS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// LSE of each row from its per-chunk (max, sum) partials, or from the caller's LSE.
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx == 0 && a.status) *a.status = 0u;   // the epilogue, later on the stream, sets bits
  if (idx >= (int64_t)a.n_lg * a.rows) return;
  const int lg = (int)(idx / a.rows);
  const int row = (int)(idx - (int64_t)lg * a.rows);
  int64_t nat;
  const float lse2 = row_lse2(a, lg, row, &nat);
  a.lse2[idx] = lse2;
  if (nat >= 0 && a.lse_out) a.lse_out[nat] = (float)((double)lse2 * 0.6931471805599453);
}

}  // namespace

hipError_t launch_score_pass(const ScoreArgs& a, bool pass2, hipStream_t s) {
  const int group_rows = a.rows < kRowsPerGroup ? a.rows : kRowsPerGroup;
  const int nw = (group_rows + 31) / 32;
  if (trace_on())
    trace_launch("%s grid=%lld block=%d  layers=%d kv_heads=%d tokens=%lld rows=%d row_groups=%d chunk=%d chunks=%d%s%s",
                 pass2 ? "mass_pass" : "lse_pass",
                 (long long)a.n_chunks * a.n_rsplit * a.n_kv_heads * a.n_layers, nw * 64, a.n_layers, a.n_kv_heads,
                 (long long)a.n_tokens, a.rows, a.n_rsplit, a.chunk, a.n_chunks,
                 pass2 && a.max_log ? " group_max" : "", pass2 && a.fuse_combine ? " combines_lse" : "");
  if (!pass2) return launch_nw<-1>(a, nw, s);
  switch (a.max_log) {
    case 0: return launch_nw<0>(a, nw, s);
    case 1: return launch_nw<1>(a, nw, s);
    case 2: return launch_nw<2>(a, nw, s);
    case 3: return launch_nw<3>(a, nw, s);
    case 4: return launch_nw<4>(a, nw, s);
    case 5: return launch_nw<5>(a, nw, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lse_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_lg * a.rows;
  if (trace_on())
    trace_launch("lse_combine grid=%lld block=256  rows=%lld chunks=%d%s", (long long)((n + 255) / 256), (long long)n,
                 a.n_chunks, a.lse_in ? " lse_in" : "");
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
