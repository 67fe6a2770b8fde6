/*
 * One eviction step driven from C through include/kvscore.h alone (no Python between
 * the caller and the library): H2O scoring with the foresight bonus and pinned sinks and
 * recent tokens, token selection, then compaction of the kept rows with renumbering.
 *
 * usage: c_pipeline IN_DIR OUT_DIR
 *   IN_DIR/meta.txt: n_layers n_kv_heads n_q_heads n_tokens window budget n_spans
 *                    n_sink n_recent limit rope_theta
 *   IN_DIR/k.bin, v.bin   bf16 [n_layers][pages][16][n_kv_heads][128] (pages = ceil(N/16))
 *   IN_DIR/q.bin          bf16 [n_layers][window][n_q_heads][128]
 *   IN_DIR/span_id.bin    int32 [n_tokens]
 *   IN_DIR/span_bonus.bin float32 [n_spans]
 * Writes OUT_DIR/{mass,item_score,item_pinned,keep,n_keep,status,new_pos,dst_k,dst_v}.bin.
 * Exit status 0 on success; otherwise the failing call is printed to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvscore.h"

#define HIP(x)                                                                  \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      return 2;                                                                 \
    }                                                                           \
  } while (0)
#define KV(x)                                                                   \
  do {                                                                          \
    int32_t r_ = (x);                                                           \
    if (r_ != KV_OK) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #x, kv_strerror(r_));                  \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

static void *read_file(const char *dir, const char *name, size_t want) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *buf = malloc(want ? want : 1);
  size_t got = buf ? fread(buf, 1, want, f) : 0;
  fclose(f);
  if (got != want) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return -1;
  size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

/* device copy of a host file, or NULL */
static void *upload(const char *dir, const char *name, size_t bytes) {
  void *h = read_file(dir, name, bytes);
  void *d = NULL;
  if (!h) return NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess)
    d = NULL;
  free(h);
  return d;
}

static int download(const char *dir, const char *name, const void *dev, size_t bytes) {
  void *h = malloc(bytes ? bytes : 1);
  if (!h) return -1;
  int rc = hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) == hipSuccess ? write_file(dir, name, h, bytes) : -1;
  free(h);
  return rc;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN_DIR OUT_DIR\n", argv[0]);
    return 1;
  }
  const char *in = argv[1], *out = argv[2];
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", in);
  FILE *mf = fopen(path, "r");
  if (!mf) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  int L, hkv, hq, W, n_spans, n_sink, n_recent, limit;
  long long n_ll, b_ll;
  double theta;
  int nread = fscanf(mf, "%d %d %d %lld %d %lld %d %d %d %d %lf", &L, &hkv, &hq, &n_ll, &W, &b_ll, &n_spans,
                     &n_sink, &n_recent, &limit, &theta);
  fclose(mf);
  if (nread != 11 || L <= 0 || hkv <= 0 || hq <= 0 || n_ll <= 0 || b_ll <= 0 || b_ll % 16 || n_spans <= 0) {
    fprintf(stderr, "bad meta.txt\n");
    return 1;
  }
  if (kv_abi_version() != KV_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header ABI %d\n", kv_abi_version(), KV_ABI_VERSION);
    return 1;
  }
  const int64_t N = n_ll, B = b_ll;
  const int64_t pages = (N + 15) / 16;
  const size_t slot = (size_t)hkv * 128;
  const size_t kv_bytes = (size_t)L * pages * 16 * slot * 2;
  const size_t dst_bytes = (size_t)L * B * slot * 2;

  void *k = upload(in, "k.bin", kv_bytes), *v = upload(in, "v.bin", kv_bytes);
  void *q = upload(in, "q.bin", (size_t)L * W * hq * 128 * 2);
  void *span_id = upload(in, "span_id.bin", (size_t)N * 4);
  void *span_bonus = upload(in, "span_bonus.bin", (size_t)n_spans * 4);
  if (!k || !v || !q || !span_id || !span_bonus) {
    fprintf(stderr, "cannot load the inputs\n");
    return 1;
  }
  float *accum, *mass, *item_score;
  uint8_t *item_pinned;
  int32_t *keep, *old_pos, *new_pos;
  int64_t *n_keep;
  uint32_t *status;
  void *dk, *dv;
  HIP(hipMalloc((void **)&accum, N * 4));
  HIP(hipMalloc((void **)&mass, N * 4));
  HIP(hipMalloc((void **)&item_score, N * 4));
  HIP(hipMalloc((void **)&item_pinned, N));
  HIP(hipMalloc((void **)&keep, B * 4));
  HIP(hipMalloc((void **)&old_pos, N * 4));
  HIP(hipMalloc((void **)&new_pos, B * 4));
  HIP(hipMalloc((void **)&n_keep, 8));
  HIP(hipMalloc((void **)&status, 4));
  HIP(hipMalloc(&dk, dst_bytes));
  HIP(hipMalloc(&dv, dst_bytes));
  HIP(hipMemset(accum, 0, N * 4));
  HIP(hipMemset(dk, 0, dst_bytes));
  HIP(hipMemset(dv, 0, dst_bytes));
  int32_t *pos = (int32_t *)malloc(N * 4);
  if (!pos) return 1;
  for (int64_t j = 0; j < N; ++j) pos[j] = (int32_t)j;
  HIP(hipMemcpy(old_pos, pos, N * 4, hipMemcpyHostToDevice));
  free(pos);

  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  const kv_cache_desc src = {k, v, L, hkv, 128, 16, N, pages * 16 * (int64_t)slot, 16 * (int64_t)slot, NULL};
  const kv_cache_desc dst = {dk, dv, L, hkv, 128, 16, B, B * (int64_t)slot, 16 * (int64_t)slot, NULL};

  kv_score_params p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.n_q_heads = hq;
  p.window = W;
  p.policy = KV_POLICY_H2O;
  p.item_tokens = 1;
  p.dt_steps = 1;
  p.accum = accum;
  p.span_id = (const int32_t *)span_id;
  p.span_bonus = (const float *)span_bonus;
  p.n_spans = n_spans;
  p.n_sink = n_sink;
  p.n_recent = n_recent;
  p.mass = mass;
  p.item_score = item_score;
  p.item_pinned = item_pinned;
  p.aggregate = KV_AGG_SUM;
  size_t ws_score = 0, ws_select = 0;
  KV(kv_score_workspace_size(&src, &p, &ws_score));
  KV(kv_select_workspace_size(N, &ws_select));
  void *ws1, *ws2;
  HIP(hipMalloc(&ws1, ws_score));
  HIP(hipMalloc(&ws2, ws_select));

  KV(kv_score(&src, &p, ws1, ws_score, stream));
  KV(kv_select(item_score, item_pinned, N, 1, N, B, keep, B, n_keep, status, ws2, ws_select, stream));
  KV(kv_compact_rerope(&src, &dst, keep, n_keep, B, old_pos, new_pos, 0, theta, limit, NULL, 0, stream));
  HIP(hipStreamSynchronize(stream));

  if (download(out, "mass.bin", mass, N * 4) || download(out, "item_score.bin", item_score, N * 4) ||
      download(out, "item_pinned.bin", item_pinned, N) || download(out, "keep.bin", keep, B * 4) ||
      download(out, "n_keep.bin", n_keep, 8) || download(out, "status.bin", status, 4) ||
      download(out, "new_pos.bin", new_pos, B * 4) || download(out, "dst_k.bin", dk, dst_bytes) ||
      download(out, "dst_v.bin", dv, dst_bytes)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP(hipStreamDestroy(stream));
  void *bufs[] = {k, v, q, span_id, span_bonus, accum, mass, item_score, item_pinned, keep, old_pos,
                  new_pos, n_keep, status, dk, dv, ws1, ws2};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP(hipFree(bufs[i]));
  return 0;
}
