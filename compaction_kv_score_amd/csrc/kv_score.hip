// Windowed attention mass on gfx950: the one dense contraction of the path.
//
// What is computed (MemDecay, Method: windowed attention mass averaged over heads and
// layers; ActKV Sec. 2.3 and 7.1: A = exp(q.k - LSE) recovered from the log-sum-exp;
// PACE Sec. 2: SnapKV's observation window):
//   for every layer l, KV head g and window row r = (query head h in g's GQA group,
//   window query w), s_rj = scale * <q_r, k_j> over keys j <= N - W + w;
//   pass 1: LSE_r = log sum_j exp(s_rj)   (per key chunk, combined afterwards)
//   pass 2: mass_part[l,g][j] = sum_r exp(s_rj - LSE_r)
//
// Work decomposition: one workgroup per (layer, KV head, chunk of keys).  Its waves
// each own 64 of the G*W rows and keep those rows' queries in registers as MFMA A
// operands for the whole chunk; 64-key tiles of K are staged through LDS (double
// buffered, 16-byte global loads, padded rows against bank conflicts) and shared by
// all waves as B operands of v_mfma_f32_16x16x32_bf16.  Logits stay in the fp32
// accumulators and are consumed in registers: nothing of size rows x N is stored.
//
// Exponentials use exp2 with the scale folded into c = scale * log2(e).  Pass 1 keeps
// a running reference per lane and row and rescales only when a tile's sum would leave
// the safe range (the first tile always does), so the steady state costs one fma, one
// exp and one add per logit.  All reductions have a fixed order: results do not depend
// on scheduling.
#include "kv_internal.h"

namespace kvs {

namespace {

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared pieces of both passes: query fragments in registers, K tiles through LDS.
template <int NW>
struct TileCtx {
  static constexpr int NT = NW * 64;
  static constexpr int kPieces = kTile * 16;           // 16-byte pieces per K tile
  static constexpr int PPT = (kPieces + NT - 1) / NT;  // pieces per thread

  const ScoreArgs& a;
  int tid, lane, wv, chunk_id, g, layer, lg, n_tiles, slot_stride;
  int64_t j0, j1;
  const uint16_t* kbase;

  __device__ TileCtx(const ScoreArgs& args) : a(args) {
    tid = threadIdx.x;
    lane = tid & 63;
    wv = tid >> 6;
    int bid = blockIdx.x;
    chunk_id = bid % a.n_chunks;
    bid /= a.n_chunks;
    g = bid % a.n_kv_heads;
    layer = bid / a.n_kv_heads;
    lg = layer * a.n_kv_heads + g;
    j0 = (int64_t)chunk_id * a.chunk;
    j1 = j0 + a.chunk < a.n_tokens ? j0 + a.chunk : a.n_tokens;
    n_tiles = (int)((j1 - j0 + kTile - 1) / kTile);
    slot_stride = a.n_kv_heads * kHeadDim;
    kbase = a.k + (int64_t)layer * a.layer_stride + g * kHeadDim;
  }

  // Query rows 64*wv + 16*blk + lane%16 as 16x16x32 fragments (dims 32*ks + 8*(lane/16)).
  __device__ void load_queries(bf16x8 (&qf)[4][4]) const {
    const int W = a.window;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int row = wv * 64 + blk * 16 + (lane & 15);
      if (row < a.rows) {
        const int hl = row / W;
        const int w = row - hl * W;
        const int h = g * a.group + hl;
        const uint16_t* qp =
            a.q + (((int64_t)layer * W + w) * a.n_q_heads + h) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[blk][ks] = *(const bf16x8*)(qp + 32 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[blk][ks] = bf16x8{};
      }
    }
  }

  __device__ void load_tile(int t, uint4 (&r)[PPT]) const {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (p < kPieces) {
        const int key = p >> 4;
        const int c16 = p & 15;
        const int64_t j = j0 + (int64_t)t * kTile + key;
        if (j < j1) {
          const int64_t off = token_offset(j, a.page_shift, a.page_stride, a.block_table, slot_stride);
          v = *(const uint4*)(kbase + off + c16 * 8);
        }
      }
      r[i] = v;
    }
  }

  __device__ void store_tile(uint16_t* buf, const uint4 (&r)[PPT]) const {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      if (p < kPieces) *(uint4*)&buf[(p >> 4) * kLdsStride + (p & 15) * 8] = r[i];
    }
  }

  // K fragment of keys 16*kb + lane%16, dims 32*ks + 8*(lane/16), from an LDS tile.
  __device__ bf16x8 key_frag(const uint16_t* buf, int kb, int ks) const {
    return *(const bf16x8*)&buf[(16 * kb + (lane & 15)) * kLdsStride + 32 * ks + 8 * (lane >> 4)];
  }
};

// Pass 1: per-chunk (max, sum) of 2^(c*s) for every row, computed as S^T = K Q^T so that
// each lane holds 4 query rows x 16 keys of a tile and the running softmax state is
// lane-local (4 maxima, 4 sums).
template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void lse_pass_kernel(ScoreArgs a) {
  using Ctx = TileCtx<NW>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kTile * kLdsStride];
  const Ctx x(a);
  const int lane = x.lane;
  const float c = a.c;
  const int W = a.window;
  const int64_t first_partial_key = a.n_tokens - W;  // keys above it are hidden from some rows

  bf16x8 qf[4][4];
  x.load_queries(qf);
  // this lane's query rows: 64*wv + 16*qb + lane%16
  int wq[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) wq[qb] = (x.wv * 64 + 16 * qb + (lane & 15)) % W;

  float m[4], l[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    m[qb] = -1e30f;
    l[qb] = 0.f;
  }

  uint4 pre[Ctx::PPT];
  x.load_tile(0, pre);
  x.store_tile(lds[0], pre);
  __syncthreads();

  for (int t = 0; t < x.n_tiles; ++t) {
    const uint16_t* cur = lds[t & 1];
    if (t + 1 < x.n_tiles) x.load_tile(t + 1, pre);

    // acc[kb][qb]: C[key][query], lane holds query 16*qb + lane%16, keys 16*kb + 4*(lane/16) + i
    f32x4 acc[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) acc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kf = x.key_frag(cur, kb, ks);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          acc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], acc[kb][qb], 0, 0, 0);
      }
    }

    const int64_t tile_j0 = x.j0 + (int64_t)t * kTile;
    if (tile_j0 + kTile - 1 > first_partial_key) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t j = tile_j0 + 16 * kb + 4 * (lane >> 4) + i;
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            if (j >= x.j1 || j > first_partial_key + wq[qb]) acc[kb][qb][i] = -INFINITY;
        }
    }

    float ts[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float s = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += exp2f_fast(__builtin_fmaf(acc[kb][qb][i], c, -m[qb]));
      ts[qb] = s;
    }
    const float mx = fmaxf(fmaxf(ts[0], ts[1]), fmaxf(ts[2], ts[3]));
    // rescale when a tile sum left [0, 2^64]; always on the first tile (m = -1e30)
    if (__builtin_amdgcn_ballot_w64(!(mx <= 0x1p64f)) != 0) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, acc[kb][qb][i] * c);
        const float mn = fmaxf(m[qb], tmax);
        l[qb] *= exp2f_fast(m[qb] - mn);
        m[qb] = mn;
        float s = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s += exp2f_fast(__builtin_fmaf(acc[kb][qb][i], c, -mn));
        ts[qb] = s;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) l[qb] += ts[qb];

    if (t + 1 < x.n_tiles) x.store_tile(lds[(t + 1) & 1], pre);
    __syncthreads();
  }

  // combine the 4 lanes holding the same query (lane, lane^16, lane^32, lane^48)
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[qb], off);
      const float lo = __shfl_xor(l[qb], off);
      const float mn = fmaxf(m[qb], mo);
      l[qb] = l[qb] * exp2f_fast(m[qb] - mn) + lo * exp2f_fast(mo - mn);
      m[qb] = mn;
    }
  }
  if (lane < 16) {
    float2* out = a.lse_part + ((int64_t)x.lg * a.n_chunks + x.chunk_id) * a.rows;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int row = x.wv * 64 + 16 * qb + lane;
      if (row < a.rows) out[row] = make_float2(m[qb], l[qb]);
    }
  }
}

// Pass 2: mass_part[l,g][j] = sum over rows of 2^(c*s - lse2), computed as S = Q K^T so
// that each lane holds 16 rows x 4 keys of a tile and the per-key sums are lane-local.
template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void mass_pass_kernel(ScoreArgs a) {
  using Ctx = TileCtx<NW>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kTile * kLdsStride];
  __shared__ float colp[2][NW][kTile];
  const Ctx x(a);
  const int lane = x.lane;
  const float c = a.c;
  const int W = a.window;
  const int64_t N = a.n_tokens;
  const int64_t first_partial_key = N - W;

  bf16x8 qf[4][4];
  x.load_queries(qf);
  // C-row cr = 4*rb + i is row 64*wv + 16*rb + 4*(lane/16) + i
  float nl[16];
#pragma unroll
  for (int cr = 0; cr < 16; ++cr) {
    const int row = x.wv * 64 + (cr >> 2) * 16 + 4 * (lane >> 4) + (cr & 3);
    nl[cr] = row < a.rows ? -a.lse2[(int64_t)x.lg * a.rows + row] : -INFINITY;
  }

  uint4 pre[Ctx::PPT];
  x.load_tile(0, pre);
  x.store_tile(lds[0], pre);
  __syncthreads();

  for (int t = 0; t < x.n_tiles; ++t) {
    const int buf = t & 1;
    const uint16_t* cur = lds[buf];
    if (t + 1 < x.n_tiles) x.load_tile(t + 1, pre);

    // Two halves of 32 keys keep only half of the accumulators live.
    // acc[rb][kh]: C[row][key], lane holds key 16*(2*half+kh) + lane%16,
    // rows 16*rb + 4*(lane/16) + i
    const int64_t tile_j0 = x.j0 + (int64_t)t * kTile;
    const bool masked = tile_j0 + kTile - 1 > first_partial_key;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 acc[4][2];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) acc[rb][kh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 kf = x.key_frag(cur, 2 * half + kh, ks);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            acc[rb][kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[rb][ks], kf, acc[rb][kh], 0, 0, 0);
        }
      }
      if (masked) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int w = (x.wv * 64 + rb * 16 + 4 * (lane >> 4) + i) % W;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const int64_t j = tile_j0 + 16 * (2 * half + kh) + (lane & 15);
              if (j >= x.j1 || j > first_partial_key + w) acc[rb][kh][i] = -INFINITY;
            }
          }
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float s = 0.f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s += exp2f_fast(__builtin_fmaf(acc[rb][kh][i], c, nl[rb * 4 + i]));
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (lane < 16) colp[buf][x.wv][16 * (2 * half + kh) + lane] = s;
      }
    }

    if (t + 1 < x.n_tiles) x.store_tile(lds[buf ^ 1], pre);
    __syncthreads();

    if (x.tid < kTile) {
      const int64_t j = tile_j0 + x.tid;
      if (j < x.j1) {
        float s = colp[buf][0][x.tid];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) s += colp[buf][w2][x.tid];
        a.mass_part[(int64_t)x.lg * N + j] = s;
      }
    }
  }
}

template <bool PASS2>
hipError_t launch_nw(const ScoreArgs& a, int nw, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_chunks * a.n_kv_heads * a.n_layers));
  switch (nw) {
#define KVS_CASE(NWV)                                                              \
  case NWV:                                                                        \
    if (PASS2)                                                                     \
      hipLaunchKernelGGL((mass_pass_kernel<NWV>), grid, dim3(NWV * 64), 0, s, a);  \
    else                                                                           \
      hipLaunchKernelGGL((lse_pass_kernel<NWV>), grid, dim3(NWV * 64), 0, s, a);   \
    break;
    KVS_CASE(1)
    KVS_CASE(2)
    KVS_CASE(3)
    KVS_CASE(4)
    KVS_CASE(5)
    KVS_CASE(6)
    KVS_CASE(7)
    KVS_CASE(8)
#undef KVS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// LSE of each row from its per-chunk (max, sum) partials, or from the caller's LSE.
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.n_lg * a.rows) return;
  const int lg = (int)(idx / a.rows);
  const int row = (int)(idx - (int64_t)lg * a.rows);
  const int layer = lg / a.n_kv_heads;
  const int g = lg - layer * a.n_kv_heads;
  const int hl = row / a.window;
  const int w = row - hl * a.window;
  const int h = g * a.group + hl;
  const int64_t nat = ((int64_t)layer * a.n_q_heads + h) * a.window + w;
  float lse2;
  if (a.lse_in) {
    lse2 = (float)((double)a.lse_in[nat] * 1.4426950408889634);
  } else {
    const float2* p = a.lse_part + (int64_t)lg * a.n_chunks * a.rows + row;
    float mx = -1e30f;
    for (int ch = 0; ch < a.n_chunks; ++ch) mx = fmaxf(mx, p[(int64_t)ch * a.rows].x);
    double sum = 0.0;
    for (int ch = 0; ch < a.n_chunks; ++ch) {
      const float2 v = p[(int64_t)ch * a.rows];
      sum += (double)v.y * exp2((double)v.x - (double)mx);
    }
    lse2 = (float)((double)mx + log2(sum));
  }
  a.lse2[idx] = lse2;
  if (a.lse_out) a.lse_out[nat] = (float)((double)lse2 * 0.6931471805599453);
}

}  // namespace

hipError_t launch_score_pass(const ScoreArgs& a, bool pass2, hipStream_t s) {
  const int nw = (a.rows + 63) / 64;
  return pass2 ? launch_nw<true>(a, nw, s) : launch_nw<false>(a, nw, s);
}

hipError_t launch_lse_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_lg * a.rows;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
